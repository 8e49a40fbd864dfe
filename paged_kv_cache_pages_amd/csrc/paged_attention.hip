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
//     (tokens 0..7), the second load bytes 1024..2047 (tokens 8..15).  The next page's K and V
//     are in flight while the current page is computed.
//   * QK: each lane forms 8-element partial dots with v_dot2_f32_bf16 (BF16 pairs, FP32
//     accumulate) and the 8 lanes of a token are summed with three DPP adds.
//   * Softmax in log2 units with a lazily moved anchor: scores are compared with the anchor
//     plus 8; only when a page exceeds it does the wavefront recompute the anchor and rescale
//     its accumulators (the result is independent of the anchor; fp32 holds 2^8 of headroom).
//   * PV: each lane accumulates p * V for its 8 dims and 4 heads in 32 FP32 registers; the
//     token lanes are summed once at the end.
//   * Long contexts with few (sequence, KV head) pairs are cut into partitions; each writes its
//     (max, sum, partial output) per query head and a merge kernel combines them.
// Block-table entries are read straight into a VGPR (one entry per lane) and moved to scalar
// registers with v_readlane; every entry is range-checked before a page is touched.
#include <math.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kAnchorHeadroom = 8.0f;  // log2 units

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

// Maximum over the whole wavefront of a value that is already uniform within 8-lane groups.
__device__ __forceinline__ float wave_max_of_groups(float x) {
  x = fmax_plain(x, dpp<kRowRor8>(x));
  x = fmax_plain(x, __shfl_xor(x, 16));
  x = fmax_plain(x, __shfl_xor(x, 32));
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

struct WaveState {
  float acc[kGroup][8];  // un-normalised sum of p * V for dims 8*chunk..8*chunk+7
  float lsum[kGroup];    // sum of p over this lane's token slots
  float m[kGroup];       // softmax anchor (log2 units), uniform across the wavefront
  float thr[kGroup];     // anchor + headroom: a score above it moves the anchor
};

// One page: K rows in ka (tokens 0..7) / kb (tokens 8..15), V rows likewise.  `valid` is the
// number of tokens of the page inside the context (only the last page can be partial).
template <bool kPartial>
__device__ __forceinline__ void process_page(WaveState &st, const uint32_t (&qv)[kGroup][4], uint4 ka, uint4 kb,
                                             uint4 va, uint4 vb, int tok, int valid, float c_log2) {
  float sa[kGroup], sb[kGroup];
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    float x = dot2_bf16(qv[h][0], ka.x, 0.0f);
    x = dot2_bf16(qv[h][1], ka.y, x);
    x = dot2_bf16(qv[h][2], ka.z, x);
    x = dot2_bf16(qv[h][3], ka.w, x);
    float y = dot2_bf16(qv[h][0], kb.x, 0.0f);
    y = dot2_bf16(qv[h][1], kb.y, y);
    y = dot2_bf16(qv[h][2], kb.z, y);
    y = dot2_bf16(qv[h][3], kb.w, y);
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
    if (!a_ok) va = make_uint4(0u, 0u, 0u, 0u);
    if (!b_ok) vb = make_uint4(0u, 0u, 0u, 0u);
  }

  float smax[kGroup];
  bool over = false;
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    smax[h] = fmax_plain(sa[h], sb[h]);
    over |= smax[h] > st.thr[h];
  }
  if (__any(over)) {
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      const float page_max = wave_max_of_groups(smax[h]);
      const float m_new = fmax_plain(st.m[h], page_max);
      const float alpha = __builtin_amdgcn_exp2f(st.m[h] - m_new);  // 0 on the first page
#pragma unroll
      for (int d = 0; d < 8; ++d) st.acc[h][d] *= alpha;
      st.lsum[h] *= alpha;
      st.m[h] = m_new;
      st.thr[h] = m_new + kAnchorHeadroom;
    }
  }

  float fa[8], fb[8];
  fa[0] = bf16_lo(va.x); fa[1] = bf16_hi(va.x); fa[2] = bf16_lo(va.y); fa[3] = bf16_hi(va.y);
  fa[4] = bf16_lo(va.z); fa[5] = bf16_hi(va.z); fa[6] = bf16_lo(va.w); fa[7] = bf16_hi(va.w);
  fb[0] = bf16_lo(vb.x); fb[1] = bf16_hi(vb.x); fb[2] = bf16_lo(vb.y); fb[3] = bf16_hi(vb.y);
  fb[4] = bf16_lo(vb.z); fb[5] = bf16_hi(vb.z); fb[6] = bf16_lo(vb.w); fb[7] = bf16_hi(vb.w);
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    const float pa = __builtin_amdgcn_exp2f(sa[h] - st.m[h]);
    const float pb = __builtin_amdgcn_exp2f(sb[h] - st.m[h]);
    st.lsum[h] += pa + pb;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      st.acc[h][d] = __builtin_fmaf(pa, fa[d], st.acc[h][d]);
      st.acc[h][d] = __builtin_fmaf(pb, fb[d], st.acc[h][d]);
    }
  }
}

__device__ __forceinline__ uint4 load16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

template <bool kSplit, bool kOutBf16>
__global__ __launch_bounds__(kThreads) void paged_decode_kernel(DecodeParams p) {
  __shared__ float s_acc[kWaves][4][kGroup][kHeadDim];  // [wave][16-lane row][head][dim]
  __shared__ float s_l[kWaves][4][kGroup];
  __shared__ float s_m[kWaves][kGroup];
  __shared__ int s_bad[kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = blockIdx.x % p.num_parts;
  const int pair = blockIdx.x / p.num_parts;
  const int g = pair % p.num_kv_heads;
  const int b = pair / p.num_kv_heads;
  const int qh0 = g * kGroup;  // first query head of the group

  const int L = p.context_lens[b];
  const bool len_ok = L >= 0 && L <= p.max_blocks * kBlock;
  const int n_pages = len_ok ? (L + kBlock - 1) / kBlock : 0;
  const int p0 = part * p.part_pages;
  const int p1 = min(p0 + p.part_pages, n_pages);

  if (p0 >= p1) {
    if (kSplit) return;  // empty partition (or empty/invalid sequence): the merge handles it
    // Empty or invalid sequence: zeros for the group's 4 x 64 outputs.
    const int64_t o = ((int64_t)b * p.num_q_heads + qh0) * kHeadDim + threadIdx.x;
    if (kOutBf16) static_cast<uint16_t *>(p.out)[o] = 0;
    else static_cast<float *>(p.out)[o] = 0.0f;
    return;
  }

  const int tok = lane >> 3;    // token within each half page
  const int chunk = lane & 7;   // 16-byte chunk of the row: dims 8*chunk .. 8*chunk+7
  const float c_log2 = p.score_log2;

  uint32_t qv[kGroup][4];
  {
    const uint16_t *qb = p.q + ((int64_t)b * p.num_q_heads + qh0) * kHeadDim + chunk * 8;
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      const uint4 t = load16(qb + h * kHeadDim);
      qv[h][0] = t.x; qv[h][1] = t.y; qv[h][2] = t.z; qv[h][3] = t.w;
    }
  }

  WaveState st;
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
#pragma unroll
    for (int d = 0; d < 8; ++d) st.acc[h][d] = 0.0f;
    st.lsum[h] = 0.0f;
    st.m[h] = -INFINITY;
    st.thr[h] = -INFINITY;
  }

  // Pages of this wavefront: p0 + wave + kWaves * k for k < n_w.
  int n_w = (p1 - p0 - wave + kWaves - 1) / kWaves;
  if (n_w < 0) n_w = 0;
  const int32_t *bt = p.block_tables + (int64_t)b * p.max_blocks + p0 + wave;
  const int64_t head_elems = (int64_t)kBlock * kHeadDim;
  const int64_t page_elems = (int64_t)p.num_kv_heads * head_elems;
  const uint16_t *kbase = p.k_pool + g * head_elems + lane * 8;
  const uint16_t *vbase = p.v_pool + g * head_elems + lane * 8;
  bool bad = false;

  // Page ids for local pages [base, base + 64): one per lane, all range-checked.
  auto fetch_ids = [&](int base, int &ids) -> bool {
    const int k = base + lane;
    const int id = k < n_w ? bt[(int64_t)kWaves * k] : 0;
    ids = id;
    return __any(id < 0 || id >= p.num_pages);
  };

  int ids = 0;
  uint4 ka = make_uint4(0u, 0u, 0u, 0u), kb = ka, va = ka, vb = ka;
  if (n_w > 0) {
    if (fetch_ids(0, ids)) {
      bad = true;
      n_w = 0;
    } else {
      const int64_t off = (int64_t)__builtin_amdgcn_readfirstlane(ids) * page_elems;
      ka = load16(kbase + off);
      kb = load16(kbase + off + 512);
      va = load16(vbase + off);
      vb = load16(vbase + off + 512);
    }
  }

  for (int k = 0; k < n_w; ++k) {
    uint4 nka = ka, nkb = kb, nva = va, nvb = vb;
    const int kn = k + 1;
    if (kn < n_w) {
      if ((kn & 63) == 0 && fetch_ids(kn, ids)) {
        bad = true;
        n_w = kn;  // stop after this page; the group's output will be zeroed
      } else {
        const int64_t off = (int64_t)__builtin_amdgcn_readlane(ids, kn & 63) * page_elems;
        nka = load16(kbase + off);
        nkb = load16(kbase + off + 512);
        nva = load16(vbase + off);
        nvb = load16(vbase + off + 512);
      }
    }
    const int page_idx = p0 + wave + kWaves * k;
    const int valid = L - page_idx * kBlock;
    if (valid >= kBlock) process_page<false>(st, qv, ka, kb, va, vb, tok, valid, c_log2);
    else process_page<true>(st, qv, ka, kb, va, vb, tok, valid, c_log2);
    ka = nka; kb = nkb; va = nva; vb = nvb;
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
    const int64_t slot = ((int64_t)b * p.num_q_heads + qh0 + h) * p.num_parts + part;
    p.part_o[slot * kHeadDim + d] = O;
    if (d == 0) {
      p.part_ml[slot * 2 + 0] = M;
      p.part_ml[slot * 2 + 1] = Ls;
    }
  } else {
    const float r = any_bad ? 0.0f : O / Ls;
    const int64_t o = ((int64_t)b * p.num_q_heads + qh0 + h) * kHeadDim + d;
    if (kOutBf16) static_cast<uint16_t *>(p.out)[o] = f32_to_bf16_rne(r);
    else static_cast<float *>(p.out)[o] = r;
  }
}

// Combine the partitions of one (sequence, query head): M = max m_i, O = sum o_i 2^(m_i - M),
// l = sum l_i 2^(m_i - M), out = O / l.  The sequence's table row is re-validated here, so an
// invalid entry anywhere zeroes the row exactly as the unsplit kernel does.
template <bool kOutBf16>
__global__ __launch_bounds__(64) void merge_partitions_kernel(DecodeParams p) {
  const int b = blockIdx.x / p.num_q_heads;
  const int h = blockIdx.x % p.num_q_heads;
  const int d = threadIdx.x;
  const int L = p.context_lens[b];
  const bool len_ok = L > 0 && L <= p.max_blocks * kBlock;
  const int n_pages = len_ok ? (L + kBlock - 1) / kBlock : 0;
  bool bad = false;
  const int32_t *bt = p.block_tables + (int64_t)b * p.max_blocks;
  for (int i = d; i < n_pages; i += 64) {
    const int id = bt[i];
    bad |= id < 0 || id >= p.num_pages;
  }
  bad = __any(bad);
  float r = 0.0f;
  if (len_ok && !bad) {
    const int n_parts = (n_pages + p.part_pages - 1) / p.part_pages;
    const int64_t slot0 = ((int64_t)b * p.num_q_heads + h) * p.num_parts;
    float M = -INFINITY;
    for (int i = 0; i < n_parts; ++i) M = fmax_plain(M, p.part_ml[(slot0 + i) * 2]);
    float O = 0.0f, Ls = 0.0f;
    for (int i = 0; i < n_parts; ++i) {
      const float e = __builtin_amdgcn_exp2f(p.part_ml[(slot0 + i) * 2] - M);
      O = __builtin_fmaf(e, p.part_o[(slot0 + i) * kHeadDim + d], O);
      Ls = __builtin_fmaf(e, p.part_ml[(slot0 + i) * 2 + 1], Ls);
    }
    r = O / Ls;
  }
  const int64_t o = ((int64_t)b * p.num_q_heads + h) * kHeadDim + d;
  if (kOutBf16) static_cast<uint16_t *>(p.out)[o] = f32_to_bf16_rne(r);
  else static_cast<float *>(p.out)[o] = r;
}

}  // namespace

hipError_t launch_paged_decode(const DecodeParams &p, bool out_bf16, hipStream_t stream) {
  const int64_t groups = (int64_t)p.batch * p.num_kv_heads * p.num_parts;
  if (groups == 0) return hipSuccess;
  if (groups > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)groups), block(kThreads);
  if (p.num_parts == 1) {
    if (out_bf16) hipLaunchKernelGGL((paged_decode_kernel<false, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((paged_decode_kernel<false, false>), grid, block, 0, stream, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((paged_decode_kernel<true, true>), grid, block, 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 mgrid((unsigned)((int64_t)p.batch * p.num_q_heads));
  if (out_bf16) hipLaunchKernelGGL((merge_partitions_kernel<true>), mgrid, dim3(64), 0, stream, p);
  else hipLaunchKernelGGL((merge_partitions_kernel<false>), mgrid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
