// CPU checks of the library's host-side logic, built with g++ under the
// address and undefined-behaviour sanitizers by tests/test_sanitizers.py:
// the launch planners (paged_kv_cache_05_amd/csrc/pa_plan.cpp) against
// their stated invariants on seeded random batches and at their limits, and
// the block manager (paged_kv_cache_05_amd/csrc/pa_manager.cpp) on seeded
// random add / fork / append / free / swap programs, consistency-checked
// after every operation.  No GPU, no HIP.  Exits 0 when every check holds;
// otherwise prints the first failure and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pa_manager.h"
#include "pa_plan.h"

namespace {

int g_checks = 0;

#define CHECK(cond, ...)                                                   \
  do {                                                                     \
    ++g_checks;                                                            \
    if (!(cond)) {                                                         \
      fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond);      \
      fprintf(stderr, __VA_ARGS__);                                        \
      fprintf(stderr, "\n");                                               \
      exit(1);                                                             \
    }                                                                      \
  } while (0)

using Rng = std::mt19937_64;

int uni(Rng &r, int lo, int hi) {  // inclusive
  return std::uniform_int_distribution<int>(lo, hi)(r);
}

// A random batch of context lengths (several shapes of distribution).
std::vector<int32_t> random_lengths(Rng &r, int n, int max_ctx) {
  std::vector<int32_t> c(n);
  const int kind = uni(r, 0, 3);
  for (int i = 0; i < n; ++i) {
    switch (kind) {
      case 0: c[i] = uni(r, 0, max_ctx); break;
      case 1: c[i] = uni(r, 0, 3) == 0 ? 0 : uni(r, 1, std::max(1, max_ctx / 16)); break;
      case 2: c[i] = uni(r, 0, 9) == 0 ? max_ctx : uni(r, 1, 64); break;
      default: c[i] = uni(r, -5, max_ctx + 50); break;   // out of range: clamped
    }
  }
  return c;
}

// ---------------------------------------------------------------------------
// decode planner
// ---------------------------------------------------------------------------

void check_plan_work_once(const std::vector<int32_t> &ctx, int max_ctx, int part) {
  const int n = (int)ctx.size();
  static pa::WorkList items, merges;   // large: keep off the stack
  int waves = -1;
  const bool ok = pa::plan_work(ctx.data(), n, max_ctx, part, &items, &merges, &waves);
  // the items the plan must contain, in (sequence, partition) order
  std::vector<std::pair<uint32_t, int>> want;   // (code, tokens)
  std::vector<uint32_t> want_merge;
  long long tokens = 0;
  for (int b = 0; b < n; ++b) {
    const int c = std::min(std::max(ctx[b], 0), max_ctx);
    tokens += c;
    const int np = c == 0 ? 1 : (c + part - 1) / part;
    for (int q = 0; q < np; ++q)
      want.push_back({(uint32_t)b << 16 | (uint32_t)q, std::min(part, c - q * part)});
    if (np > 1) want_merge.push_back((uint32_t)b);
  }
  if (!ok) {
    CHECK((int)want.size() > pa::kMaxListed, "refused a plan of %zu items", want.size());
    return;
  }
  CHECK((int)want.size() <= pa::kMaxListed, "accepted %zu items", want.size());
  CHECK(items.count == (int)want.size(), "%d items, want %zu", items.count, want.size());
  // every item exactly once
  std::vector<uint32_t> got(items.item, items.item + items.count), exp;
  for (auto &w : want) exp.push_back(w.first);
  std::vector<uint32_t> gs = got, es = exp;
  std::sort(gs.begin(), gs.end());
  std::sort(es.begin(), es.end());
  CHECK(gs == es, "item sets differ");
  // merge rows: exactly the multi-partition sequences, ascending
  CHECK(std::vector<uint32_t>(merges.item, merges.item + merges.count) == want_merge,
        "merge rows differ (%d vs %zu)", merges.count, want_merge.size());
  // order: long items (> twice the mean) first, longest first, ties and the
  // rest in (sequence, partition) order
  const long long long_item = 2 * tokens / (long long)want.size();
  std::map<uint32_t, int> tok;
  for (auto &w : want) tok[w.first] = w.second;
  std::vector<std::pair<uint32_t, int>> longs, rest;
  for (auto &w : want) (w.second > long_item ? longs : rest).push_back(w);
  std::stable_sort(longs.begin(), longs.end(),
                   [](const std::pair<uint32_t, int> &a, const std::pair<uint32_t, int> &b) {
                     return a.second > b.second;
                   });
  std::vector<uint32_t> order;
  for (auto &w : longs) order.push_back(w.first);
  for (auto &w : rest) order.push_back(w.first);
  CHECK(got == order, "launch order differs");
  const int want_waves = (long long)want.size() * 192 > tokens ? 4 : 8;
  CHECK(waves == want_waves, "waves %d, want %d", waves, want_waves);
}

void check_plan_work(Rng &r) {
  const int parts[] = {16, 32, 48, 64, 128, 256, 512, 1024, 2048, 4096, 65536};
  for (int it = 0; it < 3000; ++it) {
    const int n = uni(r, 1, uni(r, 0, 4) == 0 ? 1200 : 100);
    const int max_ctx = uni(r, 0, uni(r, 0, 1) ? 2048 : 20000);
    const int part = parts[uni(r, 0, 10)];
    check_plan_work_once(random_lengths(r, n, max_ctx), max_ctx, part);
  }
  // limits of the 16-bit fields and of the list: 960 empty sequences, one
  // sequence of 960 partitions, one item over the capacity
  check_plan_work_once(std::vector<int32_t>(960, 0), 100, 16);
  check_plan_work_once(std::vector<int32_t>(961, 0), 100, 16);
  check_plan_work_once(std::vector<int32_t>(1, 960 * 16), 960 * 16, 16);
  check_plan_work_once(std::vector<int32_t>(1, 960 * 16 + 1), 960 * 16 + 1, 16);
  check_plan_work_once(std::vector<int32_t>(65535, 1), 1, 16);
}

void check_plan_partition(Rng &r) {
  for (int it = 0; it < 2000; ++it) {
    const int n = uni(r, 1, 300);
    const int H = uni(r, 1, 96);
    const int D = uni(r, 0, 1) ? 64 : 128;
    const int max_ctx = uni(r, 1, 70000);
    const std::vector<int32_t> ctx = random_lengths(r, n, max_ctx);
    const bool have_ws = uni(r, 0, 3) != 0;
    const size_t ws = have_ws ? (size_t)uni(r, 0, 1 << 28) : 0;
    const int part = pa::plan_partition(ctx.data(), n, H, D, max_ctx, ws, have_ws);
    CHECK(part == 4096 || part == 2048 || part == 1024 || part == 512 || part == 256,
          "partition %d", part);
    auto items_at = [&](int p) {
      long long items = 0;
      for (int b = 0; b < n; ++b) {
        const int c = pa::clamp_ctx(ctx[b], max_ctx);
        items += (long long)H * (c == 0 ? 1 : (c + p - 1) / p);
      }
      return items;
    };
    auto fits = [&](int p) {
      const int np = pa::num_partitions(max_ctx, p);
      return np <= 1 ||
             (have_ws && pa::decode_workspace_layout(n, H, D, np).total <= ws);
    };
    if (part < 4096) {
      CHECK(fits(part), "planned partition %d does not fit the workspace", part);
      CHECK(items_at(part * 2) < 2048, "halved below a batch with enough items");
    }
    // stopped for a reason: enough items, the minimum, or the next would not fit
    CHECK(items_at(part) >= 2048 || part == 256 || !fits(part / 2),
          "stopped at %d without a reason", part);
  }
}

void check_workspace_layout(Rng &r) {
  for (int it = 0; it < 2000; ++it) {
    const int n = uni(r, 0, 5000), H = uni(r, 1, 128), D = uni(r, 0, 1) ? 64 : 128;
    const int np = uni(r, 1, 70);
    const pa::WorkspaceLayout w = pa::decode_workspace_layout(n, H, D, np);
    const size_t parts = (size_t)n * H * np;
    CHECK(w.ml_off == 0 && w.o_off >= parts * 8 && w.o_off % 256 == 0, "ml region");
    CHECK(w.total >= w.o_off + parts * D * 4 && w.total % 256 == 0, "o region");
    CHECK(w.o_off < parts * 8 + 256 && w.total < w.o_off + parts * D * 4 + 256, "padding");
  }
}

// ---------------------------------------------------------------------------
// prefill planners
// ---------------------------------------------------------------------------

struct PrefillCase {
  std::vector<int32_t> qs, ctx;
  int max_ctx, max_q;
};

PrefillCase random_prefill(Rng &r) {
  PrefillCase c;
  const int n = uni(r, 1, uni(r, 0, 4) == 0 ? 400 : 24);
  c.qs.push_back(0);
  c.max_ctx = 0;
  c.max_q = 0;
  for (int b = 0; b < n; ++b) {
    const int m = uni(r, 0, 5) == 0 ? 0 : uni(r, 1, uni(r, 0, 1) ? 300 : 5000);
    const int prefix = uni(r, 0, 2) == 0 ? uni(r, 0, 8000) : 0;
    c.qs.push_back(c.qs.back() + m);
    c.ctx.push_back(prefix + m);
    c.max_ctx = std::max(c.max_ctx, prefix + m);
    c.max_q = std::max(c.max_q, m);
  }
  return c;
}

void check_plan_prefill(Rng &r) {
  static pa::PrefillPlan plan;
  static pa::SplitList split, merges;
  for (int it = 0; it < 3000; ++it) {
    const PrefillCase c = random_prefill(r);
    const int n = (int)c.ctx.size();
    const int tile = uni(r, 0, 3) == 0 ? 64 : 128;
    const bool with_ctx = uni(r, 0, 3) != 0;
    const bool ok = pa::plan_prefill(c.qs.data(), with_ctx ? c.ctx.data() : nullptr, n,
                                     c.max_ctx, c.max_q, tile, &plan);
    // expected tiles and weights
    std::map<uint32_t, int64_t> want;
    for (int b = 0; b < n; ++b) {
      const int64_t m = c.qs[b + 1] - c.qs[b];
      if (m <= 0) continue;
      const int64_t ctx = with_ctx ? std::min<int64_t>(c.ctx[b], c.max_ctx) : m;
      const int64_t tiles = (m + tile - 1) / tile;
      for (int64_t t = 0; t < tiles; ++t)
        want[(uint32_t)b << 16 | (uint32_t)t] = ctx - m + std::min<int64_t>(m, (t + 1) * tile);
    }
    if (!ok) {
      CHECK((int)want.size() > pa::kMaxListed, "refused %zu tiles", want.size());
      continue;
    }
    CHECK(plan.count == (int)want.size(), "%d tiles, want %zu", plan.count, want.size());
    std::map<uint32_t, int64_t> got;
    for (int i = 0; i < plan.count; ++i) got[plan.item[i].code] = plan.item[i].work;
    CHECK(got == want, "tiles or weights differ");
    // grouped by sequence; sequences by heaviest tile desc (then id asc);
    // tiles of a sequence heaviest first
    std::map<uint32_t, int64_t> heaviest;
    for (auto &kv : want) {
      auto &h = heaviest[kv.first >> 16];
      h = std::max(h, kv.second);
    }
    std::set<uint32_t> seen;
    for (int i = 0; i < plan.count; ++i) {
      const uint32_t s = plan.item[i].code >> 16;
      if (i > 0) {
        const uint32_t p = plan.item[i - 1].code >> 16;
        if (p == s) {
          CHECK(plan.item[i - 1].work >= plan.item[i].work, "tiles not heaviest first");
        } else {
          CHECK(!seen.count(s), "sequence %u not contiguous", s);
          CHECK(heaviest[p] > heaviest[s] || (heaviest[p] == heaviest[s] && p < s),
                "sequence order");
        }
      }
      seen.insert(s);
    }
    // split plan on the same list
    const int H = uni(r, 1, 64);
    const int resident = uni(r, 0, 3) == 0 ? 0 : uni(r, 1, 2000);
    const int gpc = uni(r, 1, 4);
    const int ktile = uni(r, 0, 1) ? 32 : 64;
    const size_t slots = (size_t)uni(r, 0, 300);
    if (!pa::plan_prefill_split(plan, H, resident, gpc, ktile, slots, &split, &merges)) continue;
    CHECK(split.count <= pa::kMaxSplitItems && merges.count <= split.count, "split sizes");
    int e = 0, mi = 0;
    std::set<uint32_t> used_slots;
    int extra_chunks = 0;
    for (int i = 0; i < plan.count; ++i) {
      CHECK(e < split.count && split.item[e] == plan.item[i].code, "split order at %d", i);
      const uint32_t part0 = split.part[e];
      const int nc = part0 == 0 ? 1 : (int)(part0 & 15u) + 1;
      CHECK(nc >= 1 && nc <= pa::kMaxChunks, "chunks %d", nc);
      const int64_t tiles = (plan.item[i].work + ktile - 1) / ktile;
      if (nc > 1) {
        CHECK(tiles >= 48 && tiles / nc >= 16, "a short tile was split");
        const uint32_t slot0 = part0 >> 8;
        for (int c2 = 0; c2 < nc; ++c2) {
          const uint32_t p = split.part[e + c2];
          CHECK(split.item[e + c2] == plan.item[i].code, "chunk item");
          CHECK((p >> 8) == slot0 + (uint32_t)c2 && ((p >> 4) & 15u) == (uint32_t)c2 &&
                    (int)(p & 15u) == nc - 1,
                "chunk code");
          CHECK((p >> 8) < slots && used_slots.insert(p >> 8).second, "slot reused or out");
        }
        CHECK(mi < merges.count && merges.item[mi] == plan.item[i].code &&
                  merges.part[mi] == (slot0 << 8 | (uint32_t)(nc - 1)),
              "merge entry");
        ++mi;
        extra_chunks += nc - 1;
      }
      e += nc;
    }
    CHECK(e == split.count && mi == merges.count, "lists longer than the plan");
    CHECK(extra_chunks > 0, "a split plan without a split");
    CHECK((int64_t)extra_chunks * H <=
              (int64_t)resident * 2 / gpc - (int64_t)plan.count * H,
          "more chunks than idle workgroup slots");
  }
}

// ---------------------------------------------------------------------------
// block manager
// ---------------------------------------------------------------------------

void check_manager(Rng &r) {
  for (int prog = 0; prog < 60; ++prog) {
    const int B = 1 << uni(r, 0, 5);
    const int NB = uni(r, 4, 200), NH = uni(r, 0, 1) ? NB : 0;
    pa_manager *m = pa_manager_create(NB, B, NH, nullptr);
    CHECK(m != nullptr, "create");
    std::map<int64_t, int> len;        // resident sequences and their lengths
    std::set<int64_t> swapped;
    int64_t next_id = 0;
    std::vector<int64_t> pairs(2 * 4 * NB);
    for (int op = 0; op < 400; ++op) {
      const int kind = uni(r, 0, 9);
      std::vector<int64_t> live;
      for (auto &kv : len)
        if (!swapped.count(kv.first)) live.push_back(kv.first);
      if (kind <= 1 || len.empty()) {
        CHECK(pa_manager_add(m, next_id) == PA_OK, "add");
        len[next_id++] = 0;
      } else if (kind == 2 && !live.empty()) {
        const int64_t p = live[uni(r, 0, (int)live.size() - 1)];
        CHECK(pa_manager_fork(m, p, next_id) == PA_OK, "fork");
        len[next_id++] = len[p];
      } else if (kind <= 6 && !live.empty()) {
        std::vector<int64_t> seqs;
        const int k = uni(r, 1, std::min<int>(8, (int)live.size()));
        for (int i = 0; i < k; ++i) seqs.push_back(live[uni(r, 0, (int)live.size() - 1)]);
        std::vector<int64_t> slots(k);
        int np = -1;
        const int free_before = pa_manager_num_free(m);
        const int rc = pa_manager_append(m, seqs.data(), k, slots.data(), pairs.data(),
                                         (int)pairs.size() / 2, &np);
        CHECK(rc == PA_OK || rc == PA_ERR_NO_BLOCKS, "append rc %d", rc);
        if (rc == PA_OK) {
          for (int64_t s : seqs) ++len[s];
          for (int64_t s : slots) CHECK(s >= 0 && s < (int64_t)NB * B, "slot %lld", (long long)s);
          std::set<int64_t> uniq(slots.begin(), slots.end());
          CHECK((int)uniq.size() == k, "two tokens got one slot");
          for (int i = 0; i < np; ++i)
            CHECK(pairs[2 * i] != pairs[2 * i + 1] && pairs[2 * i] >= 0 &&
                      pairs[2 * i + 1] < NB,
                  "copy pair");
        } else {
          CHECK(pa_manager_num_free(m) == free_before, "a refused append changed the pool");
        }
      } else if (kind == 7) {
        std::vector<int64_t> all;
        for (auto &kv : len) all.push_back(kv.first);
        const int64_t s = all[uni(r, 0, (int)all.size() - 1)];
        CHECK(pa_manager_free(m, s) == PA_OK, "free");
        len.erase(s);
        swapped.erase(s);
      } else if (kind == 8 && NH > 0 && !live.empty()) {
        const int64_t s = live[uni(r, 0, (int)live.size() - 1)];
        int np = -1;
        const int rc = pa_manager_swap_out(m, &s, 1, pairs.data(), (int)pairs.size() / 2, &np);
        CHECK(rc == PA_OK || rc == PA_ERR_NO_BLOCKS, "swap out rc %d", rc);
        if (rc == PA_OK) swapped.insert(s);
      } else if (kind == 9 && !swapped.empty()) {
        const int64_t s = *swapped.begin();
        int np = -1;
        const int rc = pa_manager_swap_in(m, &s, 1, pairs.data(), (int)pairs.size() / 2, &np);
        CHECK(rc == PA_OK || rc == PA_ERR_NO_BLOCKS, "swap in rc %d", rc);
        if (rc == PA_OK) swapped.erase(s);
      }
      CHECK(pa_manager_check(m) == PA_OK, "manager inconsistent after op %d", op);
      CHECK(pa_manager_num_sequences(m) == (int)len.size(), "sequence count");
      for (auto &kv : len) CHECK(pa_manager_length(m, kv.first) == kv.second, "length");
    }
    // tables of the resident sequences: -1 past each one's blocks
    std::vector<int64_t> live;
    for (auto &kv : len)
      if (!swapped.count(kv.first)) live.push_back(kv.first);
    if (!live.empty()) {
      int max_blocks = 1;
      for (int64_t s : live) max_blocks = std::max(max_blocks, (len[s] + B - 1) / B);
      std::vector<int32_t> tables(live.size() * max_blocks), ctx(live.size());
      CHECK(pa_manager_tables(m, live.data(), (int)live.size(), tables.data(), max_blocks,
                              ctx.data()) == PA_OK,
            "tables");
      for (size_t i = 0; i < live.size(); ++i) {
        const int nb = (len[live[i]] + B - 1) / B;
        CHECK(ctx[i] == len[live[i]], "context length");
        for (int j = 0; j < max_blocks; ++j) {
          const int32_t t = tables[i * max_blocks + j];
          CHECK(j < nb ? (t >= 0 && t < NB) : t == -1, "table entry");
        }
      }
    }
    pa_manager_destroy(m);
  }
}

}  // namespace

int main(int argc, char **argv) {
  const uint64_t seed = argc > 1 ? strtoull(argv[1], nullptr, 10) : 12345;
  Rng r(seed);
  check_workspace_layout(r);
  check_plan_work(r);
  check_plan_partition(r);
  check_plan_prefill(r);
  check_manager(r);
  printf("plan_check ok: %d checks, seed %llu\n", g_checks, (unsigned long long)seed);
  return 0;
}
