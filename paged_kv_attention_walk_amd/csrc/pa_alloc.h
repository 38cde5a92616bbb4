// Exact fixed-block allocator of pool pages (host side).
//
// Properties (Luce-Org/lucebox pull 555, Summary: exact fixed-block
// allocator, transactional allocation, stale-handle detection, immediate
// release):
//  * exact: free + used == n_blocks; never hands out more than is free;
//  * all-or-none allocation and release;
//  * lowest free page index first (K/V pages from the bottom of the arena,
//    as ashhart/TensorFold issue 1156 does, Design / Host), which makes the
//    index sequence of any history unique and reproducible;
//  * handles carry a 32-bit generation that a successful free advances, so a
//    handle used after its page was freed is detected.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

namespace pa {

class BlockAllocator {
 public:
  enum Result { kOk = 0, kInvalid = -1, kNoMem = -2, kStale = -3 };

  explicit BlockAllocator(int32_t n_blocks);

  int32_t n_blocks() const { return n_blocks_; }
  int32_t n_free() const { return n_free_; }

  // Allocates n pages (lowest indices first) or nothing.
  Result alloc(int32_t n, uint64_t* handles, int32_t* indices);
  // Frees all handles or none; see the checks in the .cpp.
  Result free(int32_t n, const uint64_t* handles);
  // True when page `index` is currently allocated.
  bool is_allocated(int32_t index) const;
  uint32_t generation(int32_t index) const { return gen_[index]; }

 private:
  int32_t n_blocks_;
  int32_t n_free_;
  int32_t first_word_;             // no free page below 64 * first_word_
  std::vector<uint64_t> free_bits_;  // bit set = page free
  std::vector<uint32_t> gen_;
  std::vector<uint64_t> mark_;     // scratch bitmap for duplicate detection
};

}  // namespace pa
