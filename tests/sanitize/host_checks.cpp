// Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the page
// allocator (random histories against a plain model of the allocator's
// rules), the C-ABI pool lifecycle on host-only pools, the split-K plan over
// random batches, and the argument checks of every entry point with bad
// arguments.  Built by the host compiler with device_stubs.cpp in place of
// the kernels, run on the CPU; a sanitizer report aborts the run, a failed
// expectation exits with status 1.

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pa.h"
#include "pa_alloc.h"

namespace {

int g_fail = 0;

#define EXPECT(cond)                                                                     \
  do {                                                                                   \
    if (!(cond)) {                                                                       \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                                          \
    }                                                                                    \
  } while (0)

// The allocator's rules written plainly: a free flag and a generation per
// page; allocation takes the lowest free pages; a free checks every handle
// (in range, current generation, allocated, not repeated) before releasing
// any, then advances each page's generation.
struct Model {
  std::vector<bool> free_;
  std::vector<uint32_t> gen_;
  explicit Model(int n) : free_(n, true), gen_(n, 1) {}
  int n_free() const {
    int c = 0;
    for (bool f : free_) c += f;
    return c;
  }
  int alloc(int n, std::vector<uint64_t>& h) {
    if (n < 0) return -1;
    if (n > n_free()) return -2;
    for (int i = 0; i < static_cast<int>(free_.size()) && static_cast<int>(h.size()) < n; ++i)
      if (free_[i]) {
        free_[i] = false;
        h.push_back((static_cast<uint64_t>(gen_[i]) << 32) | static_cast<uint32_t>(i));
      }
    return 0;
  }
  int release(const std::vector<uint64_t>& h) {
    std::vector<bool> seen(free_.size(), false);
    for (uint64_t x : h) {
      const uint32_t idx = static_cast<uint32_t>(x), g = static_cast<uint32_t>(x >> 32);
      if (idx >= free_.size()) return -1;
      if (g != gen_[idx] || free_[idx] || seen[idx]) return -3;
      seen[idx] = true;
    }
    for (uint64_t x : h) {
      const uint32_t idx = static_cast<uint32_t>(x);
      free_[idx] = true;
      gen_[idx] = gen_[idx] == 0xFFFFFFFFu ? 1 : gen_[idx] + 1;
    }
    return 0;
  }
};

void allocator_histories() {
  const int sizes[] = {1, 5, 63, 64, 65, 130, 1000};
  for (int n_blocks : sizes) {
    for (int seed = 0; seed < 20; ++seed) {
      std::mt19937 rng(1000 * n_blocks + seed);
      pa::BlockAllocator a(n_blocks);
      Model m(n_blocks);
      std::vector<uint64_t> held;
      for (int step = 0; step < 300; ++step) {
        if (rng() % 2) {
          const int n = static_cast<int>(rng() % (n_blocks / 3 + 2)) - (rng() % 16 == 0 ? 1 : 0);
          std::vector<uint64_t> h(n > 0 ? n : 1), mh;
          std::vector<int32_t> ix(n > 0 ? n : 1);
          const int r = a.alloc(n, h.data(), ix.data());
          const int mr = m.alloc(n, mh);
          EXPECT(r == mr);
          if (r == 0) {
            for (int i = 0; i < n; ++i) {
              EXPECT(h[i] == mh[i]);
              EXPECT(ix[i] == static_cast<int32_t>(static_cast<uint32_t>(mh[i])));
              held.push_back(h[i]);
            }
          }
        } else if (!held.empty()) {
          // a random subset of held handles, sometimes with one bad handle in it
          std::vector<uint64_t> f;
          std::vector<uint64_t> keep;
          for (uint64_t x : held) (rng() % 3 == 0 ? f : keep).push_back(x);
          const int bad = rng() % 5;
          if (bad == 1 && !f.empty()) f.push_back(f[0]);                                  // repeated
          if (bad == 2) f.push_back(static_cast<uint64_t>(n_blocks + rng() % 4));         // out of range
          if (bad == 3 && !f.empty()) f.push_back(f.back() + (1ull << 32));               // stale generation
          const int r = a.free(static_cast<int32_t>(f.size()), f.data());
          const int mr = m.release(f);
          EXPECT(r == mr);
          if (r == 0) held.swap(keep);
        }
        EXPECT(a.n_free() == m.n_free());
        for (int i = 0; i < n_blocks; ++i) {
          EXPECT(a.is_allocated(i) == !m.free_[i]);
          EXPECT(a.generation(i) == m.gen_[i]);
        }
      }
    }
  }
}

pa_pool_desc host_desc(int n_blocks, int page, int32_t kv) {
  pa_pool_desc d{};
  d.n_blocks = n_blocks;
  d.page_size = page;
  d.n_kv_heads = PA_N_KV_HEADS;
  d.head_dim = PA_HEAD_DIM;
  d.kv_type = kv;
  d.flags = PA_POOL_HOST_ONLY;
  return d;
}

void pool_lifecycle() {
  std::mt19937 rng(7);
  const int32_t kvs[] = {PA_KV_TYPE(PA_Q4_0, PA_Q4_0), PA_KV_TYPE(PA_Q8_0, PA_Q4_0), PA_KV_TYPE(PA_BF16, PA_F16)};
  for (int it = 0; it < 200; ++it) {
    const int n = 1 + static_cast<int>(rng() % 300);
    const int page = 16 * (1 + static_cast<int>(rng() % 32));
    pa_pool_desc d = host_desc(n, page, kvs[it % 3]);
    pa_pool* p = nullptr;
    EXPECT(pa_pool_create(&d, &p) == PA_OK && p);
    if (!p) continue;
    pa_pool_info info{};
    EXPECT(pa_pool_get_info(p, &info) == PA_OK && info.n_free == n && info.k_pool == nullptr);
    std::vector<pa_block> h(n);
    std::vector<int32_t> ix(n);
    const int k = static_cast<int>(rng() % (n + 1));
    EXPECT(pa_alloc_blocks(p, k, h.data(), ix.data()) == PA_OK);
    EXPECT(pa_alloc_blocks(p, n - k + 1, h.data(), nullptr) == PA_ERR_NOMEM);
    EXPECT(pa_free_blocks(p, k, h.data()) == PA_OK);
    EXPECT(pa_free_blocks(p, k > 0 ? 1 : 0, h.data()) == (k > 0 ? PA_ERR_STALE : PA_OK));
    EXPECT(pa_pool_get_info(p, &info) == PA_OK && info.n_free == n);
    // host-only pools have no device side
    const int32_t blk = 0, slot = 0;
    std::vector<uint8_t> row(4 * 512, 0);
    EXPECT(pa_append_kv(p, 1, &blk, &slot, row.data(), row.data(), nullptr) == PA_ERR_INVALID);
    EXPECT(pa_pool_destroy(p) == PA_OK);
  }
  // bad descriptors
  pa_pool* p = nullptr;
  pa_pool_desc d = host_desc(0, 16, PA_KV_TYPE(PA_Q4_0, PA_Q4_0));
  EXPECT(pa_pool_create(&d, &p) == PA_ERR_INVALID && !p);
  d = host_desc(8, 40, PA_KV_TYPE(PA_Q4_0, PA_Q4_0));
  EXPECT(pa_pool_create(&d, &p) == PA_ERR_UNSUPPORTED && !p);
  d = host_desc(8, 16, PA_KV_TYPE(PA_Q4_0, PA_Q4_0));
  d.head_dim = 128;
  EXPECT(pa_pool_create(&d, &p) == PA_ERR_INVALID && !p);
  d = host_desc(8, 16, 0x10000 | PA_Q4_0);
  EXPECT(pa_pool_create(&d, &p) != PA_OK && !p);
  EXPECT(pa_pool_create(nullptr, &p) == PA_ERR_INVALID);
  EXPECT(pa_pool_destroy(nullptr) == PA_OK);
}

void split_plans() {
  std::mt19937 rng(11);
  std::vector<int32_t> lens(PA_HOST_PLAN_MAX_SEQS), first(PA_HOST_PLAN_MAX_SEQS + 1);
  for (int it = 0; it < 3000; ++it) {
    const int n_seq = static_cast<int>(rng() % (PA_HOST_PLAN_MAX_SEQS + 1));
    const int cap = 16 * (1 + static_cast<int>(rng() % 20000));
    for (int s = 0; s < n_seq; ++s) {
      const int r = static_cast<int>(rng() % 20);
      lens[s] = r == 0 ? -static_cast<int32_t>(rng() % 5) - 1
                       : r == 1 ? cap + 1 + static_cast<int32_t>(rng() % 100)
                                : static_cast<int32_t>(rng() % (static_cast<uint32_t>(cap) + 1));
    }
    const int n_cu = 1 + static_cast<int>(rng() % 512), wgs = 1 + static_cast<int>(rng() % 4);
    int32_t chunk = -1, items = -1;
    EXPECT(pa_split_plan(lens.data(), n_seq, cap, n_cu, wgs, &chunk, &items, first.data()) == PA_OK);
    if (n_seq == 0) {
      EXPECT(chunk == 0 && items == 0 && first[0] == 0);
      continue;
    }
    EXPECT(chunk > 0 && chunk % 128 == 0);
    EXPECT(first[0] == 0 && items == PA_N_KV_HEADS * first[n_seq]);
    for (int s = 0; s < n_seq; ++s) {
      const int L = lens[s];
      const int want = (L <= 0 || L > cap) ? 1 : (L + chunk - 1) / chunk;
      EXPECT(first[s + 1] - first[s] == want);
    }
  }
  int32_t c = 0, n = 0;
  EXPECT(pa_split_plan(lens.data(), PA_HOST_PLAN_MAX_SEQS + 1, 64, 1, 1, &c, &n, nullptr) == PA_ERR_INVALID);
  EXPECT(pa_split_plan(nullptr, 3, 64, 1, 1, &c, &n, nullptr) == PA_ERR_INVALID);
  EXPECT(pa_split_plan(lens.data(), 3, 0, 1, 1, &c, &n, nullptr) == PA_ERR_INVALID);
  EXPECT(pa_split_plan(lens.data(), 3, 64, 0, 1, &c, &n, nullptr) == PA_ERR_INVALID);
  EXPECT(pa_split_plan(lens.data(), 3, 64, 1, 0, &c, &n, nullptr) == PA_ERR_INVALID);
  EXPECT(pa_split_plan(lens.data(), 3, 64, 1, 1, nullptr, &n, nullptr) == PA_ERR_INVALID);
}

// Fake device addresses that are never dereferenced: every call here fails
// in a host check, or (with a plausible workspace) at the first device step.
void entry_point_checks() {
  const uintptr_t base = 1u << 20;
  const float* q = reinterpret_cast<const float*>(base);
  const void* kp = reinterpret_cast<const void*>(base);
  const int32_t* bt = reinterpret_cast<const int32_t*>(base);
  float* out = reinterpret_cast<float*>(base);
  const int32_t kv = PA_KV_TYPE(PA_Q4_0, PA_Q4_0);
  auto dec = [&](const float* qq, const void* k, int32_t n_seq, int32_t T, int32_t kvt, int32_t page, float* o,
                 const pa_decode_ext* e) { return pa_decode(qq, k, k, bt, bt, n_seq, T, kvt, page, o, nullptr, e); };
  EXPECT(dec(q, kp, 1, 0, kv, 16, out, nullptr) == PA_ERR_INVALID);
  EXPECT(dec(q, kp, 1, 9, kv, 16, out, nullptr) == PA_ERR_INVALID);
  EXPECT(dec(q, kp, -1, 1, kv, 16, out, nullptr) == PA_ERR_INVALID);
  EXPECT(dec(q, kp, 1, 1, 0x10000 | PA_Q4_0, 16, out, nullptr) == PA_ERR_INVALID);
  EXPECT(dec(q, kp, 1, 1, kv, 40, out, nullptr) == PA_ERR_UNSUPPORTED);
  EXPECT(dec(q + 1, kp, 1, 1, kv, 16, out, nullptr) == PA_ERR_INVALID);
  EXPECT(dec(q, kp, 1, 1, kv, 16, nullptr, nullptr) == PA_ERR_INVALID);
  EXPECT(dec(q, kp, 1, 1, kv, 16, out, nullptr) == PA_ERR_NOT_FOUND);
  EXPECT(dec(q, kp, 0, 1, kv, 16, out, nullptr) == PA_OK);
  pa_decode_ext e{};
  EXPECT(dec(q, kp, 1, 1, kv, 16, out, &e) == PA_ERR_INVALID);              // bt_stride 0
  e.bt_stride = 4;
  e.n_pool_blocks = 8;
  e.flags = 2;
  EXPECT(dec(q, kp, 1, 1, kv, 16, out, &e) == PA_ERR_INVALID);              // unknown flag
  // plausible calls with a host plan: the plan is computed, then the device
  // step fails (no device here)
  std::vector<int32_t> lens = {0, 1, 17, 4000, 64, 63};
  for (int T = 1; T <= PA_MAX_QTOK; ++T) {
    size_t ws = 0;
    EXPECT(pa_decode_workspace_size(static_cast<int32_t>(lens.size()), T, 0, &ws) == PA_OK && ws > 0);
    pa_decode_ext x{};
    x.bt_stride = 256;
    x.n_pool_blocks = 1024;
    x.workspace = reinterpret_cast<void*>(base);
    x.workspace_bytes = ws;
    x.seq_lens_host = lens.data();
    const pa_status st = dec(q, kp, static_cast<int32_t>(lens.size()), T, kv, 16, out, &x);
    EXPECT(st != PA_OK && st != PA_ERR_INVALID);
    x.workspace_bytes = ws - 1;
    EXPECT(dec(q, kp, static_cast<int32_t>(lens.size()), T, kv, 16, out, &x) == PA_ERR_INVALID);
  }
  size_t b = 0;
  EXPECT(pa_decode_workspace_size(-1, 1, 0, &b) == PA_ERR_INVALID);
  EXPECT(pa_decode_workspace_size(1, 9, 0, &b) == PA_ERR_INVALID);
  EXPECT(pa_decode_workspace_size(1, 1, 0, nullptr) == PA_ERR_INVALID);
  EXPECT(pa_prefill_workspace_size(1, 0, 0, &b) == PA_ERR_INVALID);
  EXPECT(pa_prefill_workspace_size(1, PA_MAX_PREFILL_TOKENS + 1, 0, &b) == PA_ERR_INVALID);
  EXPECT(pa_prefill(q, kp, kp, bt, bt, 1, 0, kv, 16, out, nullptr, nullptr) == PA_ERR_INVALID);
  EXPECT(pa_prefill(q, kp, kp, bt, bt, 1, 100, kv, 16, out, nullptr, nullptr) == PA_ERR_NOT_FOUND);
  // appends without a pool, probes and queries with bad arguments
  EXPECT(pa_append_kv(nullptr, 1, bt, bt, kp, kp, nullptr) == PA_ERR_INVALID);
  EXPECT(pa_append_kv_device(nullptr, 1, bt, bt, kp, kp, PA_F32, nullptr, nullptr) == PA_ERR_INVALID);
  uint32_t* sink = reinterpret_cast<uint32_t*>(base);
  EXPECT(pa_read_bandwidth_probe_ex(kp, 0, sink, 1 << 20, 8, 1, 0, nullptr) == PA_ERR_INVALID);
  EXPECT(pa_read_bandwidth_probe_ex(kp, 24, sink, 1 << 20, 8, 1, 0, nullptr) == PA_ERR_INVALID);
  EXPECT(pa_read_bandwidth_probe_ex(kp, 1 << 20, sink, 1 << 20, 0, 1, 0, nullptr) == PA_ERR_INVALID);
  EXPECT(pa_read_bandwidth_probe_ex(kp, 1 << 20, sink, 1 << 20, 8, 3, 0, nullptr) == PA_ERR_INVALID);
  EXPECT(pa_read_bandwidth_probe_ex(kp, 1 << 20, sink, 1 << 20, 8, 1, 4, nullptr) == PA_ERR_INVALID);
  EXPECT(pa_read_bandwidth_probe_ex(kp, 1 << 20, sink, 1, 8, 1, 0, nullptr) == PA_ERR_INVALID);
  int32_t w = 0;
  EXPECT(pa_split_workgroups_per_cu(kv, 0, 0, &w) == PA_ERR_INVALID);
  EXPECT(pa_split_workgroups_per_cu(kv, 1, 2, &w) == PA_ERR_INVALID);
  EXPECT(pa_split_workgroups_per_cu(kv, 1, 0, nullptr) == PA_ERR_INVALID);
  int32_t err = 0;
  EXPECT(pa_get_device_error(nullptr, nullptr, nullptr, 0, nullptr) == PA_ERR_INVALID);
  EXPECT(pa_get_device_error(nullptr, nullptr, nullptr, 0, &err) != PA_OK);
  EXPECT(pa_row_bytes(PA_Q4_0) == 144 && pa_row_bytes(PA_Q8_0) == 272 && pa_row_bytes(99) == 0);
  for (int st = -7; st <= 1; ++st) EXPECT(pa_status_string(st) != nullptr);
}

}  // namespace

int main() {
  allocator_histories();
  pool_lifecycle();
  split_plans();
  entry_point_checks();
  if (g_fail) {
    std::fprintf(stderr, "%d expectation(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
