// Host-side validation of block tables, positions and context lengths (plain C++, no GPU).
//
// The pages' host code asserts when it meets an impossible page-table state instead of
// continuing ("The prefill path: flowing the entire prompt at once", section "Distributing K/V into paged blocks"); the
// library's equivalent is this opt-in check, run before launching when PKV_DEBUG_VALIDATE=1 and
// callable directly on host arrays.
#include <stdint.h>

#include <unordered_set>

#include "pagedkv.h"

namespace {
constexpr int kBlock = 16;
}

extern "C" pkv_status pkv_validate_append_host(const int32_t *block_tables, int32_t max_blocks_per_seq,
                                               const int32_t *positions, int32_t batch, int32_t num_pages,
                                               int32_t *bad_row) {
  if (bad_row) *bad_row = -1;
  if (batch < 0 || max_blocks_per_seq <= 0 || num_pages <= 0) return PKV_ERR_SHAPE;
  if (batch == 0) return PKV_OK;
  if (!block_tables || !positions) return PKV_ERR_NULL;
  std::unordered_set<int64_t> targets;
  targets.reserve((size_t)batch * 2);
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t pos = positions[b];
    bool ok = pos >= 0 && (int64_t)pos < (int64_t)max_blocks_per_seq * kBlock;
    int32_t page = -1;
    if (ok) {
      page = block_tables[(int64_t)b * max_blocks_per_seq + pos / kBlock];
      ok = page >= 0 && page < num_pages;
    }
    if (ok) ok = targets.insert((int64_t)page * kBlock + pos % kBlock).second;  // distinct targets
    if (!ok) {
      if (bad_row) *bad_row = b;
      return PKV_ERR_VALIDATION;
    }
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_validate_decode_host(const int32_t *block_tables, int32_t max_blocks_per_seq,
                                               const int32_t *context_lens, int32_t batch, int32_t num_pages,
                                               int32_t *bad_row) {
  if (bad_row) *bad_row = -1;
  if (batch < 0 || max_blocks_per_seq <= 0 || num_pages <= 0) return PKV_ERR_SHAPE;
  if (batch == 0) return PKV_OK;
  if (!block_tables || !context_lens) return PKV_ERR_NULL;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t L = context_lens[b];
    bool ok = L >= 0 && (int64_t)L <= (int64_t)max_blocks_per_seq * kBlock;
    const int32_t n = ok ? (L + kBlock - 1) / kBlock : 0;
    for (int32_t j = 0; ok && j < n; ++j) {
      const int32_t page = block_tables[(int64_t)b * max_blocks_per_seq + j];
      ok = page >= 0 && page < num_pages;
    }
    if (!ok) {
      if (bad_row) *bad_row = b;
      return PKV_ERR_VALIDATION;
    }
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_validate_prefill_host(const int32_t *block_tables, int32_t max_blocks_per_seq,
                                                const int32_t *cu_seqlens, const int32_t *start_pos, int32_t batch,
                                                int32_t num_tokens, int32_t max_prompt_len, int32_t num_pages,
                                                int32_t *bad_row) {
  if (bad_row) *bad_row = -1;
  if (batch < 0 || num_tokens < 0 || max_prompt_len < 0 || max_blocks_per_seq <= 0 || num_pages <= 0)
    return PKV_ERR_SHAPE;
  if (batch == 0) return PKV_OK;
  if (!block_tables || !cu_seqlens || !start_pos) return PKV_ERR_NULL;
  std::unordered_set<int64_t> targets;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t row0 = cu_seqlens[b], end = cu_seqlens[b + 1], start = start_pos[b];
    const int64_t n = end - row0;
    bool ok = row0 >= 0 && n >= 0 && end <= num_tokens && n <= max_prompt_len && start >= 0 &&
              start + n <= (int64_t)max_blocks_per_seq * kBlock;
    if (ok) {
      const int32_t *row = block_tables + (int64_t)b * max_blocks_per_seq;
      const int64_t need = (start + n + kBlock - 1) / kBlock;
      for (int64_t e = 0; ok && e < need; ++e) ok = row[e] >= 0 && row[e] < num_pages;
      for (int64_t pos = start; ok && pos < start + n; ++pos)
        ok = targets.insert((int64_t)row[pos / kBlock] * kBlock + pos % kBlock).second;
    }
    if (!ok) {
      if (bad_row) *bad_row = b;
      return PKV_ERR_VALIDATION;
    }
  }
  return PKV_OK;
}

// A BF16 value is finite unless its 8 exponent bits are all ones (infinity or NaN).
extern "C" pkv_status pkv_validate_finite_rows_host(const uint16_t *rows, int32_t num_rows, int32_t row_elems,
                                                    int32_t *bad_row) {
  if (bad_row) *bad_row = -1;
  if (num_rows < 0 || row_elems <= 0) return PKV_ERR_SHAPE;
  if (num_rows == 0) return PKV_OK;
  if (!rows) return PKV_ERR_NULL;
  for (int32_t r = 0; r < num_rows; ++r) {
    const uint16_t *row = rows + (int64_t)r * row_elems;
    for (int32_t i = 0; i < row_elems; ++i) {
      if ((row[i] & 0x7F80u) == 0x7F80u) {
        if (bad_row) *bad_row = r;
        return PKV_ERR_VALIDATION;
      }
    }
  }
  return PKV_OK;
}
