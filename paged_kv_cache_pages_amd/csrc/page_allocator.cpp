// Host page allocator with admission credits (plain C++, no GPU).
//
// Admission reserves, per request, the pages of its longest stored prefix in every layer and
// admits first-in-first-out while those credits fit beside the active requests' ("6 Hours of
// YouTube and 85 handtyped pages of notes on LLM Inference", section "Current scope").  Physical
// pages are taken lazily from the back of a free list when a block is first needed ("The
// prefill path: flowing the entire prompt at once", section "Distributing K/V into paged
// blocks").  Because a request never takes more pages than its credits, and the active
// requests' credits never exceed the pool, an admitted request always finds its pages: the
// decode loop cannot deadlock on page growth and nothing is ever preempted.
//
// The tables are kept in exactly the int32 [layer][block] layout the kernels read, so a decode
// step's tables are row copies.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

namespace {

constexpr int32_t kBlock = 16;

struct Waiting {
  int64_t id;
  int64_t credits;
};

struct Active {
  int64_t credits = 0;
  int64_t assigned = 0;
  std::vector<int32_t> table;  // [layer][block], -1 = unassigned
};

int64_t pages_for(int64_t tokens) { return (tokens + kBlock - 1) / kBlock; }

}  // namespace

struct pkv_allocator {
  int32_t num_pages = 0;
  int32_t layers = 0;
  int32_t max_blocks = 0;
  int64_t context = 0;
  bool static_batching = false;
  std::vector<int32_t> free_list;  // taken from and returned to the back
  std::deque<Waiting> waiting;
  std::unordered_map<int64_t, Active> active;
  int64_t credits_reserved = 0;
  pkv_alloc_stats stats{};

  int64_t credits_for(int32_t prompt, int32_t max_new) const {
    // The last generated token is returned, never appended: the longest stored prefix is
    // prompt + allowed - 1 tokens, and at least the prompt itself.
    const int64_t allowed = std::max<int64_t>(0, std::min<int64_t>(max_new, context - prompt));
    const int64_t prefix = std::max<int64_t>(prompt, prompt + allowed - 1);
    return (int64_t)layers * pages_for(prefix);
  }

  bool known(int64_t id) const {
    if (active.count(id)) return true;
    for (const Waiting &w : waiting)
      if (w.id == id) return true;
    return false;
  }

  void note_assigned() {
    const int64_t assigned = (int64_t)num_pages - (int64_t)free_list.size();
    stats.peak_assigned = std::max(stats.peak_assigned, assigned);
  }
};

extern "C" pkv_status pkv_alloc_create(int32_t num_pages, int32_t layers, int32_t max_blocks_per_seq,
                                       const int32_t *free_order, int32_t static_batching, pkv_allocator **out) {
  if (!out) return PKV_ERR_NULL;
  *out = nullptr;
  if (num_pages <= 0 || layers <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  pkv_allocator *a = new (std::nothrow) pkv_allocator();
  if (!a) return PKV_ERR_SHAPE;
  a->num_pages = num_pages;
  a->layers = layers;
  a->max_blocks = max_blocks_per_seq;
  a->context = (int64_t)max_blocks_per_seq * kBlock;
  a->static_batching = static_batching != 0;
  a->free_list.resize(num_pages);
  if (free_order) {
    std::vector<uint8_t> seen(num_pages, 0);
    for (int32_t i = 0; i < num_pages; ++i) {
      const int32_t p = free_order[i];
      if (p < 0 || p >= num_pages || seen[p]) {
        delete a;
        return PKV_ERR_SHAPE;
      }
      seen[p] = 1;
      a->free_list[i] = p;
    }
  } else {
    for (int32_t i = 0; i < num_pages; ++i) a->free_list[i] = i;
  }
  a->stats.pool_pages = num_pages;
  *out = a;
  return PKV_OK;
}

extern "C" void pkv_alloc_destroy(pkv_allocator *alloc) { delete alloc; }

extern "C" pkv_status pkv_alloc_submit(pkv_allocator *a, int64_t request_id, int32_t prompt_tokens,
                                       int32_t max_new_tokens) {
  if (!a) return PKV_ERR_NULL;
  if (a->known(request_id)) return PKV_ERR_STATE;
  if (prompt_tokens <= 0 || prompt_tokens > a->context || max_new_tokens < 0) {
    ++a->stats.rejected;
    return PKV_ERR_REJECTED;
  }
  const int64_t credits = a->credits_for(prompt_tokens, max_new_tokens);
  if (credits > a->num_pages) {  // could never fit, even alone
    ++a->stats.rejected;
    return PKV_ERR_REJECTED;
  }
  a->waiting.push_back({request_id, credits});
  return PKV_OK;
}

extern "C" pkv_status pkv_alloc_admit(pkv_allocator *a, int64_t *admitted, int32_t capacity, int32_t *count) {
  if (!a || !count) return PKV_ERR_NULL;
  *count = 0;
  if (capacity < 0) return PKV_ERR_SHAPE;
  if (capacity > 0 && !admitted) return PKV_ERR_NULL;
  int32_t n = 0;
  bool blocked = false;
  if (a->static_batching && !a->active.empty()) {
    blocked = !a->waiting.empty();
  } else {
    while (!a->waiting.empty() && n < capacity) {
      const Waiting w = a->waiting.front();
      if (a->credits_reserved + w.credits > a->num_pages) {
        blocked = true;
        break;
      }
      a->waiting.pop_front();
      Active &r = a->active[w.id];
      r.credits = w.credits;
      r.assigned = 0;
      r.table.assign((size_t)a->layers * a->max_blocks, -1);
      a->credits_reserved += w.credits;
      admitted[n++] = w.id;
    }
  }
  if (blocked) ++a->stats.admission_waits;
  a->stats.peak_active = std::max<int64_t>(a->stats.peak_active, (int64_t)a->active.size());
  *count = n;
  return PKV_OK;
}

extern "C" pkv_status pkv_alloc_ensure(pkv_allocator *a, int64_t request_id, int32_t pos) {
  if (!a) return PKV_ERR_NULL;
  auto it = a->active.find(request_id);
  if (it == a->active.end()) return PKV_ERR_STATE;
  if (pos < 0 || pos >= a->context) return PKV_ERR_SHAPE;
  Active &r = it->second;
  const int32_t blk = pos / kBlock;
  int64_t missing = 0;
  for (int32_t l = 0; l < a->layers; ++l) missing += r.table[(size_t)l * a->max_blocks + blk] < 0;
  if (missing == 0) return PKV_OK;
  // Within credits, the free list always holds the pages (credits of active requests never exceed
  // the pool); the second test only guards that invariant.
  if (r.assigned + missing > r.credits || missing > (int64_t)a->free_list.size()) return PKV_ERR_EXHAUSTED;
  for (int32_t l = 0; l < a->layers; ++l) {
    int32_t &e = r.table[(size_t)l * a->max_blocks + blk];
    if (e < 0) {
      e = a->free_list.back();
      a->free_list.pop_back();
    }
  }
  r.assigned += missing;
  a->note_assigned();
  return PKV_OK;
}

extern "C" pkv_status pkv_alloc_prepare_step(pkv_allocator *a, const int64_t *request_ids, const int32_t *positions,
                                             int32_t batch, int32_t *block_tables, int32_t *bad_row) {
  if (bad_row) *bad_row = -1;
  if (!a) return PKV_ERR_NULL;
  if (batch < 0) return PKV_ERR_SHAPE;
  if (batch > 0 && (!request_ids || !positions || !block_tables)) return PKV_ERR_NULL;
  for (int32_t b = 0; b < batch; ++b) {
    const pkv_status st = pkv_alloc_ensure(a, request_ids[b], positions[b]);
    if (st != PKV_OK) {
      if (bad_row) *bad_row = b;
      return st;
    }
  }
  const size_t row = (size_t)a->max_blocks;
  for (int32_t b = 0; b < batch; ++b) {
    const Active &r = a->active.find(request_ids[b])->second;
    for (int32_t l = 0; l < a->layers; ++l)
      memcpy(block_tables + ((size_t)l * batch + b) * row, r.table.data() + (size_t)l * row, row * sizeof(int32_t));
  }
  a->stats.largest_batch = std::max<int64_t>(a->stats.largest_batch, batch);
  return PKV_OK;
}

extern "C" pkv_status pkv_alloc_table(const pkv_allocator *a, int64_t request_id, int32_t *dst) {
  if (!a || !dst) return PKV_ERR_NULL;
  auto it = a->active.find(request_id);
  if (it == a->active.end()) return PKV_ERR_STATE;
  memcpy(dst, it->second.table.data(), it->second.table.size() * sizeof(int32_t));
  return PKV_OK;
}

extern "C" pkv_status pkv_alloc_release(pkv_allocator *a, int64_t request_id) {
  if (!a) return PKV_ERR_NULL;
  auto it = a->active.find(request_id);
  if (it == a->active.end()) return PKV_ERR_STATE;
  for (int32_t e : it->second.table)
    if (e >= 0) a->free_list.push_back(e);
  a->credits_reserved -= it->second.credits;
  a->active.erase(it);
  return PKV_OK;
}

extern "C" pkv_status pkv_alloc_get_stats(const pkv_allocator *a, pkv_alloc_stats *out) {
  if (!a || !out) return PKV_ERR_NULL;
  *out = a->stats;
  out->pool_pages = a->num_pages;
  out->free_pages = (int64_t)a->free_list.size();
  out->credits_reserved = a->credits_reserved;
  out->active = (int64_t)a->active.size();
  out->waiting = (int64_t)a->waiting.size();
  return PKV_OK;
}
