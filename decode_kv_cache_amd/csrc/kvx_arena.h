// Range sub-allocator behind the plan work lists: byte ranges carved out of
// large chunks that are never given back.  First fit over an
// address-ordered free list; a released range merges with free neighbours
// of the same chunk (never across chunks, even when two chunks happen to be
// adjacent in the address space).  Thread-safe.  It never touches the memory
// it hands out, so it holds no device code and no HIP types: the caller
// supplies the function that obtains a chunk.
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <iterator>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

namespace kvx {

class RangeArena {
 public:
  // Obtains a chunk of `bytes`; returns 0 on success, else an error code
  // that alloc passes back.
  using ChunkFn = int (*)(size_t bytes, void** out);

  RangeArena(size_t min_chunk, size_t chunk_align) : min_chunk_(min_chunk), chunk_align_(chunk_align) {}

  // A range of exactly n bytes (the caller rounds n as it needs).
  int alloc(size_t n, ChunkFn get_chunk, void** out) {
    std::lock_guard<std::mutex> lk(mu_);
    for (auto it = free_.begin(); it != free_.end(); ++it) {
      if (it->second.size < n) continue;
      const uintptr_t a = it->first;
      const Range r = it->second;
      free_.erase(it);
      if (r.size > n) free_.emplace(a + n, Range{r.size - n, r.chunk});
      *out = reinterpret_cast<void*>(a);
      return 0;
    }
    const size_t cs = std::max(min_chunk_, (n + chunk_align_ - 1) / chunk_align_ * chunk_align_);
    void* base = nullptr;
    const int rc = get_chunk(cs, &base);
    if (rc != 0) return rc;
    const int id = int(chunks_.size());
    chunks_.emplace_back(uintptr_t(base), cs);
    if (cs > n) free_.emplace(uintptr_t(base) + n, Range{cs - n, id});
    *out = base;
    return 0;
  }

  // Give back a range obtained from alloc with the same n.  False (and no
  // change) when p lies in no chunk of this arena.
  bool release(void* p, size_t n) {
    std::lock_guard<std::mutex> lk(mu_);
    const uintptr_t a = uintptr_t(p);
    int id = -1;
    for (size_t c = 0; c < chunks_.size(); ++c)
      if (a >= chunks_[c].first && a < chunks_[c].first + chunks_[c].second) id = int(c);
    if (id < 0) return false;
    auto next = free_.lower_bound(a);
    if (next != free_.end() && next->first == a + n && next->second.chunk == id) {
      n += next->second.size;
      next = free_.erase(next);
    }
    if (next != free_.begin()) {
      auto prev = std::prev(next);
      if (prev->first + prev->second.size == a && prev->second.chunk == id) {
        prev->second.size += n;
        return true;
      }
    }
    free_.emplace(a, Range{n, id});
    return true;
  }

  // For tests: free ranges, free bytes and chunk bytes.
  size_t free_ranges() {
    std::lock_guard<std::mutex> lk(mu_);
    return free_.size();
  }
  size_t free_bytes() {
    std::lock_guard<std::mutex> lk(mu_);
    size_t b = 0;
    for (const auto& f : free_) b += f.second.size;
    return b;
  }
  size_t chunk_bytes() {
    std::lock_guard<std::mutex> lk(mu_);
    size_t b = 0;
    for (const auto& c : chunks_) b += c.second;
    return b;
  }
  size_t chunks() {
    std::lock_guard<std::mutex> lk(mu_);
    return chunks_.size();
  }

 private:
  struct Range {
    size_t size;
    int chunk;
  };
  const size_t min_chunk_, chunk_align_;
  std::mutex mu_;
  std::map<uintptr_t, Range> free_;                   // start address -> free range
  std::vector<std::pair<uintptr_t, size_t>> chunks_;  // (base, bytes)
};

}  // namespace kvx
