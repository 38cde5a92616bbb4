#include "pa_alloc.h"

namespace pa {

namespace {
constexpr uint32_t kGenStart = 1;
inline uint32_t next_gen(uint32_t g) { return g == 0xFFFFFFFFu ? kGenStart : g + 1; }
}  // namespace

BlockAllocator::BlockAllocator(int32_t n_blocks)
    : n_blocks_(n_blocks), n_free_(n_blocks), first_word_(0),
      free_bits_((n_blocks + 63) / 64, ~0ull), gen_(n_blocks, kGenStart),
      mark_((n_blocks + 63) / 64, 0ull) {
  const int tail = n_blocks % 64;
  if (tail) free_bits_.back() = (1ull << tail) - 1;
}

bool BlockAllocator::is_allocated(int32_t index) const {
  if (index < 0 || index >= n_blocks_) return false;
  return !((free_bits_[index >> 6] >> (index & 63)) & 1ull);
}

BlockAllocator::Result BlockAllocator::alloc(int32_t n, uint64_t* handles, int32_t* indices) {
  if (n < 0) return kInvalid;
  if (n > n_free_) return kNoMem;          // nothing changes
  int32_t got = 0;
  size_t w = static_cast<size_t>(first_word_);
  while (got < n) {
    uint64_t bits = free_bits_[w];
    while (bits && got < n) {
      const int b = __builtin_ctzll(bits);
      bits &= bits - 1;
      const int32_t idx = static_cast<int32_t>(w * 64 + b);
      free_bits_[w] &= ~(1ull << b);
      if (handles) handles[got] = (static_cast<uint64_t>(gen_[idx]) << 32) | static_cast<uint32_t>(idx);
      if (indices) indices[got] = idx;
      ++got;
    }
    if (got < n) ++w;
  }
  n_free_ -= n;
  while (first_word_ < static_cast<int32_t>(free_bits_.size()) && free_bits_[first_word_] == 0) ++first_word_;
  return kOk;
}

BlockAllocator::Result BlockAllocator::free(int32_t n, const uint64_t* handles) {
  if (n < 0 || (n > 0 && !handles)) return kInvalid;
  // Validate everything first; `mark_` records pages seen in this call.
  Result res = kOk;
  int32_t checked = 0;
  for (; checked < n; ++checked) {
    const uint64_t h = handles[checked];
    const uint32_t idx = static_cast<uint32_t>(h & 0xFFFFFFFFu);
    const uint32_t g = static_cast<uint32_t>(h >> 32);
    if (idx >= static_cast<uint32_t>(n_blocks_)) { res = kInvalid; break; }
    const uint64_t bit = 1ull << (idx & 63);
    if (g != gen_[idx] || (free_bits_[idx >> 6] & bit) || (mark_[idx >> 6] & bit)) { res = kStale; break; }
    mark_[idx >> 6] |= bit;
  }
  // Clear the marks set so far (on success, every handle's page).
  for (int32_t i = 0; i < checked; ++i) {
    const uint32_t idx = static_cast<uint32_t>(handles[i] & 0xFFFFFFFFu);
    mark_[idx >> 6] &= ~(1ull << (idx & 63));
  }
  if (res != kOk) return res;
  for (int32_t i = 0; i < n; ++i) {
    const uint32_t idx = static_cast<uint32_t>(handles[i] & 0xFFFFFFFFu);
    free_bits_[idx >> 6] |= 1ull << (idx & 63);
    gen_[idx] = next_gen(gen_[idx]);
    if (static_cast<int32_t>(idx >> 6) < first_word_) first_word_ = static_cast<int32_t>(idx >> 6);
  }
  n_free_ += n;
  return kOk;
}

}  // namespace pa
