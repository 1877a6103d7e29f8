// The work-list arena (decode_kv_cache_amd/csrc/kvx_arena.h) under random
// allocations and releases, with made-up chunk addresses (the arena never
// touches the memory it hands out).  After every operation: live ranges lie
// inside chunks and never overlap, and free plus live bytes equal the chunk
// bytes.  Once everything is released, each chunk is one free range again.
// Two chunks are placed back to back in the address space, so a merge across
// chunks would show.  Prints "ok" and exits 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <map>
#include <random>
#include <vector>

#include "kvx_arena.h"

static uintptr_t g_next = uintptr_t(1) << 40;
static std::vector<std::pair<uintptr_t, size_t>> g_chunks;
static int g_fail_next = 0;

static int fake_chunk(size_t bytes, void** out) {
  if (g_fail_next) {
    g_fail_next = 0;
    return 2;  // an allocation error, passed back by alloc
  }
  const bool adjacent = g_chunks.size() % 2 == 1;  // every second chunk directly follows the previous one
  if (!adjacent) g_next += uintptr_t(1) << 30;
  *out = reinterpret_cast<void*>(g_next);
  g_chunks.emplace_back(g_next, bytes);
  g_next += bytes;
  return 0;
}

static int failures = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #c); \
      ++failures;                                                  \
      return;                                                      \
    }                                                              \
  } while (0)

static void check_state(kvx::RangeArena& a, const std::map<uintptr_t, size_t>& live) {
  size_t live_bytes = 0;
  uintptr_t end = 0;
  for (const auto& l : live) {
    CHECK(l.first >= end);  // ordered by address: no overlap with the previous range
    end = l.first + l.second;
    live_bytes += l.second;
    bool inside = false;
    for (const auto& c : g_chunks) inside |= l.first >= c.first && end <= c.first + c.second;
    CHECK(inside);
  }
  CHECK(a.free_bytes() + live_bytes == a.chunk_bytes());
}

static void run(uint64_t seed) {
  const size_t kMin = size_t(1) << 20, kAlign = size_t(64) << 10;
  kvx::RangeArena a(kMin, kAlign);
  std::mt19937_64 rng(seed);
  std::map<uintptr_t, size_t> live;
  for (int step = 0; step < 4000; ++step) {
    const bool do_alloc = live.empty() || rng() % 100 < 55;
    if (do_alloc) {
      size_t n = 256 * (1 + rng() % 64);  // up to 16 KiB
      if (rng() % 50 == 0) n = 256 * (1 + rng() % 8192);  // up to 2 MiB: larger than the minimum chunk
      if (rng() % 400 == 0) {
        g_fail_next = 1;
        void* p = nullptr;
        // larger than every chunk so far, so it needs a new chunk, whose allocation fails
        CHECK(a.alloc(a.chunk_bytes() + kMin, fake_chunk, &p) == 2);
        g_fail_next = 0;
        check_state(a, live);
        continue;
      }
      void* p = nullptr;
      CHECK(a.alloc(n, fake_chunk, &p) == 0);
      live.emplace(uintptr_t(p), n);
    } else {
      auto it = live.begin();
      std::advance(it, long(rng() % live.size()));
      CHECK(a.release(reinterpret_cast<void*>(it->first), it->second));
      live.erase(it);
    }
    check_state(a, live);
    if (failures) return;
  }
  for (const auto& l : live) CHECK(a.release(reinterpret_cast<void*>(l.first), l.second));
  live.clear();
  check_state(a, live);
  CHECK(a.free_ranges() == a.chunks());  // every chunk is whole again, none merged with its neighbour
  int dummy = 0;
  CHECK(!a.release(&dummy, 256));        // an address from no chunk is refused
  CHECK(a.free_ranges() == a.chunks());
}

int main() {
  for (uint64_t seed = 1; seed <= 20 && !failures; ++seed) {
    g_chunks.clear();
    run(seed);
  }
  if (failures) return 1;
  std::printf("ok\n");
  return 0;
}
