// Host-code stress driver run under AddressSanitizer and UndefinedBehaviorSanitizer (built and run by
// tests/test_host_sanitizers.py with g++; no GPU).  It drives the page allocator and the host
// validators of libpagedkv with seeded random operations, including out-of-range and hostile
// arguments, and checks the allocator's bookkeeping invariants after every operation:
//   free + held pages = pool, no page held twice, every held page a valid id, credits within the
//   pool and every active request's held pages within its credits.
// Exit status 0 when every check holds (and the sanitizers found nothing).
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <set>
#include <vector>

#include "pagedkv.h"

namespace {

int failures = 0;
// Operations that succeeded, so the caller can see the streams reached every path.
long n_submit = 0, n_admit = 0, n_step = 0, n_step_fail = 0, n_release = 0, n_exhausted = 0, n_prefill_bad = 0;

void check(bool ok, const char *what, int64_t step) {
  if (!ok) {
    if (failures < 20) fprintf(stderr, "step %lld: %s\n", (long long)step, what);
    ++failures;
  }
}

struct Active {
  int64_t id;
  int32_t prompt, max_new, pos;
};

void allocator_stream(uint32_t seed, int32_t num_pages, int32_t layers, int32_t max_blocks, bool static_batching,
                      int steps) {
  std::mt19937 rng(seed);
  std::vector<int32_t> order(num_pages);
  for (int32_t i = 0; i < num_pages; ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  pkv_allocator *a = nullptr;
  if (pkv_alloc_create(num_pages, layers, max_blocks, order.data(), static_batching ? 1 : 0, &a) != PKV_OK) {
    check(false, "create", -1);
    return;
  }
  const int32_t ctx = 16 * max_blocks;
  std::vector<Active> active;
  std::vector<int64_t> queued;
  int64_t next_id = 1;
  std::vector<int32_t> table((size_t)layers * max_blocks);
  for (int step = 0; step < steps; ++step) {
    const int op = (int)(rng() % 100);
    if (op < 25) {  // submit, sometimes with hostile sizes or a duplicate id
      int32_t prompt = 1 + (int32_t)(rng() % ctx), max_new = (int32_t)(rng() % 300);
      int64_t id = next_id++;
      const int bad = (int)(rng() % 20);
      if (bad == 0) prompt = 0;
      if (bad == 1) prompt = ctx + 1 + (int32_t)(rng() % 100);
      if (bad == 2) max_new = -1 - (int32_t)(rng() % 5);
      if (bad == 3 && !queued.empty()) id = queued[rng() % queued.size()];
      if (bad == 4) prompt = INT32_MAX;
      const pkv_status st = pkv_alloc_submit(a, id, prompt, max_new);
      if (st == PKV_OK) queued.push_back(id), ++n_submit;
      check(st == PKV_OK || st == PKV_ERR_REJECTED || st == PKV_ERR_STATE, "submit status", step);
    } else if (op < 40) {  // admit
      int64_t ids[64];
      int32_t count = -1;
      const int32_t cap = (int32_t)(rng() % 65);
      const pkv_status st = pkv_alloc_admit(a, ids, cap, &count);
      check(st == PKV_OK && count >= 0 && count <= cap, "admit", step);
      for (int32_t i = 0; st == PKV_OK && i < count; ++i) {
        queued.erase(std::remove(queued.begin(), queued.end(), ids[i]), queued.end());
        // the prompt length is not returned: take the pages for a short prefix, then grow
        active.push_back({ids[i], 1, 0, 0});
        ++n_admit;
      }
    } else if (op < 70 && !active.empty()) {  // decode step over every active request
      std::vector<int64_t> ids;
      std::vector<int32_t> pos;
      for (auto &r : active) {
        r.pos = std::min(r.pos + 1 + (int32_t)(rng() % 40), ctx + 5);  // may run past the context
        ids.push_back(r.id);
        pos.push_back(r.pos);
      }
      if (rng() % 10 == 0) pos[rng() % pos.size()] = -3;  // a bad position
      if (rng() % 10 == 0) ids[rng() % ids.size()] = -77;  // an unknown id
      std::vector<int32_t> tables((size_t)layers * ids.size() * max_blocks, 12345);
      int32_t bad_row = -2;
      const pkv_status st = pkv_alloc_prepare_step(a, ids.data(), pos.data(), (int32_t)ids.size(), tables.data(), &bad_row);
      check(st == PKV_OK ? bad_row == -1 : (bad_row >= 0 && bad_row < (int32_t)ids.size()), "prepare_step row", step);
      ++(st == PKV_OK ? n_step : n_step_fail);
      if (st == PKV_OK) {
        for (int32_t v : tables) check(v == -1 || (v >= 0 && v < num_pages), "table entry range", step);
      }
      // validators on the produced tables (host pointers), with some damage
      if (st == PKV_OK && !ids.empty()) {
        std::vector<int32_t> layer0(tables.begin(), tables.begin() + ids.size() * max_blocks);
        std::vector<int32_t> lens(pos);
        for (auto &l : lens) l += 1;
        int32_t row = -9;
        (void)pkv_validate_append_host(layer0.data(), max_blocks, pos.data(), (int32_t)ids.size(), num_pages, &row);
        (void)pkv_validate_decode_host(layer0.data(), max_blocks, lens.data(), (int32_t)ids.size(), num_pages, &row);
        layer0[rng() % layer0.size()] = (int32_t)(rng() % 3 == 0 ? -5 : num_pages + 3);
        lens[rng() % lens.size()] = (int32_t)(rng() % 2 ? -1 : 16 * max_blocks + 1);
        (void)pkv_validate_decode_host(layer0.data(), max_blocks, lens.data(), (int32_t)ids.size(), num_pages, &row);
      }
    } else if (op < 85 && !active.empty()) {  // release one
      const size_t i = rng() % active.size();
      check(pkv_alloc_release(a, active[i].id) == PKV_OK, "release", step);
      ++n_release;
      active.erase(active.begin() + i);
      check(pkv_alloc_release(a, -1234) == PKV_ERR_STATE, "release unknown", step);
    } else if (!active.empty()) {  // ensure at a random position, read a table
      const Active &r = active[rng() % active.size()];
      const int32_t pos = (int32_t)(rng() % (ctx + 20)) - 10;
      const pkv_status st = pkv_alloc_ensure(a, r.id, pos);
      check(st == PKV_OK || st == PKV_ERR_SHAPE || st == PKV_ERR_EXHAUSTED, "ensure status", step);
      n_exhausted += st == PKV_ERR_EXHAUSTED;
      check(pkv_alloc_table(a, r.id, table.data()) == PKV_OK, "table", step);
    }
    // invariants
    pkv_alloc_stats s;
    check(pkv_alloc_get_stats(a, &s) == PKV_OK, "stats", step);
    std::set<int32_t> held;
    int64_t held_count = 0;
    for (const auto &r : active) {
      if (pkv_alloc_table(a, r.id, table.data()) != PKV_OK) {
        check(false, "table of an active request", step);
        continue;
      }
      for (int32_t v : table) {
        if (v < 0) continue;
        check(v < num_pages, "held page id", step);
        check(held.insert(v).second, "page held twice", step);
        ++held_count;
      }
    }
    check(s.free_pages + held_count == num_pages, "free + held = pool", step);
    check(s.credits_reserved >= 0 && s.credits_reserved <= (int64_t)num_pages, "credits within the pool", step);
    check(s.active == (int64_t)active.size(), "active count", step);
  }
  for (const auto &r : active) pkv_alloc_release(a, r.id);
  pkv_alloc_stats s;
  pkv_alloc_get_stats(a, &s);
  check(s.free_pages == num_pages && s.credits_reserved == 0, "everything returned", steps);
  pkv_alloc_destroy(a);
}

void hostile_arguments() {
  pkv_allocator *a = nullptr;
  const int32_t dup[4] = {0, 1, 1, 3};
  check(pkv_alloc_create(0, 1, 8, nullptr, 0, &a) != PKV_OK, "create 0 pages", -1);
  check(pkv_alloc_create(4, 1, 8, dup, 0, &a) != PKV_OK, "create with a duplicate free page", -1);
  const int32_t out_of_range[4] = {0, 1, 2, 9};
  check(pkv_alloc_create(4, 1, 8, out_of_range, 0, &a) != PKV_OK, "create with an out-of-range page", -1);
  int32_t row = 0;
  const int32_t bt[2] = {0, 1};
  const int32_t pos[1] = {0};
  check(pkv_validate_append_host(bt, 2, pos, 1, 2, &row) == PKV_OK && row == -1, "validate ok", -1);
  check(pkv_validate_prefill_host(bt, 2, nullptr, nullptr, 0, 0, 0, 2, &row) == PKV_OK, "prefill, empty batch", -1);
}

// Random prefill layouts, some of them broken, through the prefill validator.
void prefill_validation(uint32_t seed, int rounds) {
  std::mt19937 rng(seed);
  for (int r = 0; r < rounds; ++r) {
    const int32_t batch = 1 + (int32_t)(rng() % 12), max_blocks = 1 + (int32_t)(rng() % 40);
    const int32_t num_pages = batch * max_blocks + (int32_t)(rng() % 8);
    std::vector<int32_t> bt((size_t)batch * max_blocks), cu(batch + 1), start(batch);
    for (size_t i = 0; i < bt.size(); ++i) bt[i] = (int32_t)i;
    std::shuffle(bt.begin(), bt.end(), rng);
    int32_t max_len = 0;
    for (int32_t b = 0; b < batch; ++b) {
      start[b] = (int32_t)(rng() % (16 * max_blocks));
      const int32_t room = 16 * max_blocks - start[b];
      const int32_t len = (int32_t)(rng() % (room + 1));
      cu[b + 1] = cu[b] + len;
      max_len = std::max(max_len, len);
    }
    const int damage = (int)(rng() % 8);
    if (damage == 0) start[rng() % batch] = -1 - (int32_t)(rng() % 5);
    if (damage == 1) bt[rng() % bt.size()] = (int32_t)(rng() % 2 ? -1 : num_pages + 2);
    if (damage == 2 && batch > 1) std::swap(cu[1], cu[batch]);
    if (damage == 3) start[rng() % batch] = 16 * max_blocks + (int32_t)(rng() % 100);
    if (damage == 4) bt[rng() % bt.size()] = bt[rng() % bt.size()];  // two rows share a page
    int32_t row = -9;
    const pkv_status st = pkv_validate_prefill_host(bt.data(), max_blocks, cu.data(), start.data(), batch, cu[batch],
                                                    max_len, num_pages, &row);
    check(st == PKV_OK ? row == -1 : (st == PKV_ERR_VALIDATION && row >= 0 && row < batch) || st == PKV_ERR_SHAPE,
          "prefill validation result", r);
    if (damage >= 5) check(st == PKV_OK, "an undamaged prefill layout validates", r);
    n_prefill_bad += st != PKV_OK;
  }
}

}  // namespace

int main() {
  hostile_arguments();
  prefill_validation(7, 3000);
  allocator_stream(1, 64, 2, 8, false, 4000);
  allocator_stream(2, 64, 2, 8, true, 4000);
  allocator_stream(3, 300, 4, 16, false, 3000);
  allocator_stream(4, 16, 1, 4, false, 4000);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("submitted %ld admitted %ld steps %ld failed_steps %ld released %ld exhausted %ld prefill_rejected %ld\n",
         n_submit, n_admit, n_step, n_step_fail, n_release, n_exhausted, n_prefill_bad);
  printf("host sanitizer stress: all checks passed\n");
  return 0;
}
