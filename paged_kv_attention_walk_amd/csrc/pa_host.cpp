// Host side of the C ABI declared in include/pa.h: argument checks, pools and
// their allocator, the pointer registry used by pa_decode without an
// extension struct, append staging, and kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_alloc.h"
#include "pa_internal.h"

namespace {

using pa::BlockAllocator;

constexpr int kTargetPerCu = 4;      // work items per compute unit the workspace is sized for
constexpr int kDefaultMaxSeqs = 512;
constexpr int kDefaultAppendRows = 1024;
constexpr int kStagingSlots = 2;

struct Staging {
  void* host = nullptr;    // pinned
  void* dev = nullptr;
  size_t bytes = 0;
  hipEvent_t done = nullptr;    // recorded after the slot's scatter kernel
  hipEvent_t copied = nullptr;  // recorded after the slot's host-to-device copy
  bool used = false;
};

}  // namespace

struct pa_pool {
  pa_pool_desc desc{};
  int k_type = 0, v_type = 0;
  int rb_k = 0, rb_v = 0;
  bool own_k = false, own_v = false;
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
  Staging staging[kStagingSlots];
  int next_slot = 0;
  hipStream_t copy_stream = nullptr;   // the staging uploads (default priority)
  BlockAllocator alloc;
  std::mutex mu;
  explicit pa_pool(int32_t n) : alloc(n) {}
};

namespace {

std::mutex g_registry_mu;
std::map<const void*, pa_pool*> g_registry;   // K base pointer -> pool

std::mutex g_cu_mu;
std::unordered_map<int, int> g_cu_count;

// Compute units of `device` (cached).  0 on failure.
int cu_count(int device) {
  std::lock_guard<std::mutex> lk(g_cu_mu);
  auto it = g_cu_count.find(device);
  if (it != g_cu_count.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n <= 0) return 0;
  g_cu_count[device] = n;
  return n;
}

int target_items(int device) {
  const int cu = cu_count(device);
  return (cu > 0 ? cu : 256) * kTargetPerCu;
}

bool type_ok(int t) { return t >= PA_F16 && t <= PA_Q4_0; }

// Splits and checks a kv_type.  Returns PA_OK and the two encodings.
pa_status parse_kv_type(int32_t kv_type, int* k, int* v) {
  if (kv_type & ~0xFFFF) return PA_ERR_INVALID;
  const int kt = kv_type & 0xFF;
  int vt = (kv_type >> 8) & 0xFF;
  if (vt == 0) vt = kt;
  if (!type_ok(kt) || !type_ok(vt)) return PA_ERR_INVALID;
  *k = kt;
  *v = vt;
  return PA_OK;
}

bool page_size_ok(int P) { return P >= 16 && P <= 512 && P % 16 == 0; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

pa_status hip_status(hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  if (e == hipErrorOutOfMemory) return PA_ERR_NOMEM;
  return PA_ERR_HIP;
}

// Sets the device for the current thread and restores the previous one.
struct DeviceGuard {
  int prev = -1;
  bool ok = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

void free_pool_resources(pa_pool* p) {
  for (auto& s : p->staging) {
    if (s.done) {
      (void)hipEventSynchronize(s.done);
      (void)hipEventDestroy(s.done);
    }
    if (s.copied) {
      (void)hipEventSynchronize(s.copied);
      (void)hipEventDestroy(s.copied);
    }
    if (s.host) (void)hipHostFree(s.host);
    if (s.dev) (void)hipFree(s.dev);
    s = Staging{};
  }
  if (p->copy_stream) {
    (void)hipStreamSynchronize(p->copy_stream);
    (void)hipStreamDestroy(p->copy_stream);
    p->copy_stream = nullptr;
  }
  if (p->workspace) (void)hipFree(p->workspace);
  p->workspace = nullptr;
  if (p->own_k && p->desc.k_pool) (void)hipFree(p->desc.k_pool);
  if (p->own_v && p->desc.v_pool) (void)hipFree(p->desc.v_pool);
}

}  // namespace

namespace pa {

static_assert(PA_HOST_PLAN_MAX_SEQS == kHostPlanSeqs, "host plan limit of the ABI");
static_assert(sizeof(DecodeParams) <= 4096, "launch arguments stay within 4 KB");

// The device plan (plan_wg / plan_chunk) in host arithmetic.
void host_plan(const int32_t* lens, int n_seq, int cap, int target, int budget, int split, int slots, int tok_total,
               HostPlan& hp) {
  auto n_chunks = [cap](int L, int chunk) { return (L <= 0 || L > cap) ? 1 : (L + chunk - 1) / chunk; };
  auto granule = [](long long c) {
    c = (c + kChunkGranule - 1) / kChunkGranule * kChunkGranule;
    if (c < kChunkGranule) c = kChunkGranule;
    return c > (1ll << 30) ? (1ll << 30) : c;
  };
  long long total = 0, mx = 0;
  for (int i = 0; i < n_seq; ++i)
    if (lens[i] > 0 && lens[i] <= cap) {
      total += lens[i];
      mx = lens[i] > mx ? lens[i] : mx;
    }
  if (split > 0 && ragged_split(mx, total, slots)) target = split;
  long long chunk = granule((total * kKvHeads + target - 1) / target);
  if (budget > 0 && total > 0) {
    const long long c0 = granule((total * kKvHeads + budget - 1) / budget);
    if (c0 < chunk) {
      long long pick = chunk;
      for (int k = kPlanCand - 1; k >= 0; --k) {
        const long long ck = c0 + static_cast<long long>(kChunkGranule) * k;
        long long cnt = 0;
        for (int i = 0; i < n_seq; ++i) cnt += n_chunks(lens[i], static_cast<int>(ck));
        if (ck < chunk && kKvHeads * cnt <= budget) pick = ck;
      }
      chunk = pick;
    }
  }
  hp.on = 1;
  hp.chunk = static_cast<int32_t>(chunk);
  hp.any_multi = 0;
  hp.first[0] = 0;
  hp.mfirst[0] = 0;
  const int rows = kKvHeads * 6 * tok_total;              // query rows of a sequence
  for (int i = 0; i < n_seq; ++i) {
    const int nc = n_chunks(lens[i], hp.chunk);
    hp.first[i + 1] = hp.first[i] + nc;
    hp.mfirst[i + 1] = hp.mfirst[i] + merge_wgs(nc, rows);
    hp.len[i] = lens[i];
    if (nc > 1) hp.any_multi = 1;
  }
  // longest-first order when the grid takes more than one round of resident
  // workgroups
  hp.lpt = (static_cast<long long>(kKvHeads) * hp.first[n_seq] > slots) ? 1 : 0;
  hp.n_full = 0;
  for (int w = 0; w < kHostPlanSeqs / 32; ++w) hp.pmask[w] = 0;
  int order[kHostPlanSeqs], last_len[kHostPlanSeqs], n_short = 0;
  for (int i = 0; i < n_seq; ++i) {
    const int L = lens[i];
    const int nc = n_chunks(L, hp.chunk);
    const int last = (L <= 0 || L > cap) ? 0 : L - (nc - 1) * hp.chunk;   // an empty sequence: one empty chunk
    if (last == hp.chunk) {
      hp.n_full += nc;
    } else {
      hp.n_full += nc - 1;
      hp.pmask[i >> 5] |= 1u << (i & 31);
      last_len[i] = last;
      order[n_short++] = i;
    }
  }
  std::stable_sort(order, order + n_short, [&](int a, int b) { return last_len[a] > last_len[b]; });
  for (int k = 0; k < n_short; ++k) hp.ord[k] = static_cast<uint8_t>(order[k]);
}

}  // namespace pa

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID: return "invalid argument";
    case PA_ERR_NOMEM: return "out of memory (pool blocks or device memory)";
    case PA_ERR_STALE: return "stale, already free or repeated block handle";
    case PA_ERR_UNSUPPORTED: return "unsupported type, page size or shape";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_NOT_FOUND: return "pointer is not the base of a live pool";
    default: return "unknown status";
  }
}

const char* pa_version(void) { return PA_VERSION_STRING; }

size_t pa_row_bytes(int32_t t) { return static_cast<size_t>(pa::row_bytes_of(t)); }

pa_status pa_decode_workspace_size(int32_t n_seq, int32_t n_qtok, int32_t device, size_t* bytes) {
  if (!bytes || n_seq < 0 || n_qtok < 1 || n_qtok > PA_MAX_QTOK) return PA_ERR_INVALID;
  *bytes = pa::workspace_layout_items(pa::max_work_items(n_seq, target_items(device)), n_qtok).total;
  return PA_OK;
}

pa_status pa_pool_create(const pa_pool_desc* d, pa_pool** out) {
  if (!d || !out) return PA_ERR_INVALID;
  if (d->n_blocks < 1 || d->n_kv_heads != PA_N_KV_HEADS || d->head_dim != PA_HEAD_DIM) return PA_ERR_INVALID;
  if (d->max_seqs < 0 || d->max_blocks_per_seq < 0 || d->max_append_rows < 0) return PA_ERR_INVALID;
  if (d->flags & ~PA_POOL_HOST_ONLY) return PA_ERR_INVALID;
  if (!page_size_ok(d->page_size)) return PA_ERR_UNSUPPORTED;
  int kt = 0, vt = 0;
  const pa_status ts = parse_kv_type(d->kv_type, &kt, &vt);
  if (ts != PA_OK) return ts;
  const bool host_only = (d->flags & PA_POOL_HOST_ONLY) != 0;
  if (!host_only && ((d->k_pool && !aligned(d->k_pool, 16)) || (d->v_pool && !aligned(d->v_pool, 16))))
    return PA_ERR_INVALID;

  pa_pool* p = new (std::nothrow) pa_pool(d->n_blocks);
  if (!p) return PA_ERR_NOMEM;
  p->desc = *d;
  p->k_type = kt;
  p->v_type = vt;
  p->rb_k = pa::row_bytes_of(kt);
  p->rb_v = pa::row_bytes_of(vt);
  if (p->desc.max_seqs == 0) p->desc.max_seqs = kDefaultMaxSeqs;
  if (p->desc.max_blocks_per_seq == 0) p->desc.max_blocks_per_seq = d->n_blocks;
  if (p->desc.max_append_rows == 0) p->desc.max_append_rows = kDefaultAppendRows;
  if (host_only) {
    p->desc.k_pool = p->desc.v_pool = nullptr;
    *out = p;
    return PA_OK;
  }

  DeviceGuard dg(d->device);
  if (!dg.ok) {
    delete p;
    return PA_ERR_INVALID;
  }
  pa_status st = PA_OK;
  const size_t kbytes = static_cast<size_t>(d->n_blocks) * PA_N_KV_HEADS * d->page_size * p->rb_k;
  const size_t vbytes = static_cast<size_t>(d->n_blocks) * PA_N_KV_HEADS * d->page_size * p->rb_v;
  if (!p->desc.k_pool) {
    st = hip_status(hipMalloc(&p->desc.k_pool, kbytes));
    p->own_k = st == PA_OK;
  }
  if (st == PA_OK && !p->desc.v_pool) {
    st = hip_status(hipMalloc(&p->desc.v_pool, vbytes));
    p->own_v = st == PA_OK;
  }
  if (st == PA_OK) {
    const pa::WorkspaceLayout wl = pa::workspace_layout(p->desc.max_seqs, target_items(d->device), PA_MAX_QTOK);
    p->workspace_bytes = wl.total;
    st = hip_status(hipMalloc(&p->workspace, p->workspace_bytes));
    if (st == PA_OK) st = hip_status(hipMemset(p->workspace, 0, wl.lse_off));   // error word
  }
  const size_t sbytes = pa::staging_bytes(p->desc.max_append_rows, p->rb_k, p->rb_v);
  for (int i = 0; st == PA_OK && i < kStagingSlots; ++i) {
    Staging& s = p->staging[i];
    s.bytes = sbytes;
    st = hip_status(hipHostMalloc(&s.host, sbytes, hipHostMallocDefault));
    if (st == PA_OK) st = hip_status(hipMalloc(&s.dev, sbytes));
    if (st == PA_OK) st = hip_status(hipEventCreateWithFlags(&s.done, hipEventDisableTiming));
    if (st == PA_OK) st = hip_status(hipEventCreateWithFlags(&s.copied, hipEventDisableTiming));
  }
  if (st == PA_OK) st = hip_status(hipStreamCreateWithFlags(&p->copy_stream, hipStreamNonBlocking));
  if (st == PA_OK) {
    std::lock_guard<std::mutex> lk(g_registry_mu);
    if (g_registry.count(p->desc.k_pool)) st = PA_ERR_INVALID;
    else g_registry[p->desc.k_pool] = p;
  }
  if (st != PA_OK) {
    free_pool_resources(p);
    delete p;
    return st;
  }
  *out = p;
  return PA_OK;
}

pa_status pa_pool_destroy(pa_pool* p) {
  if (!p) return PA_OK;
  if (p->desc.k_pool) {
    std::lock_guard<std::mutex> lk(g_registry_mu);
    auto it = g_registry.find(p->desc.k_pool);
    if (it != g_registry.end() && it->second == p) g_registry.erase(it);
  }
  if (!(p->desc.flags & PA_POOL_HOST_ONLY)) {
    DeviceGuard dg(p->desc.device);
    free_pool_resources(p);
  }
  delete p;
  return PA_OK;
}

pa_status pa_pool_get_info(const pa_pool* p, pa_pool_info* info) {
  if (!p || !info) return PA_ERR_INVALID;
  pa_pool* mp = const_cast<pa_pool*>(p);
  std::lock_guard<std::mutex> lk(mp->mu);
  std::memset(info, 0, sizeof(*info));
  info->k_pool = p->desc.k_pool;
  info->v_pool = p->desc.v_pool;
  info->workspace = p->workspace;
  info->workspace_bytes = p->workspace_bytes;
  info->k_row_bytes = p->rb_k;
  info->v_row_bytes = p->rb_v;
  info->k_page_bytes = static_cast<size_t>(PA_N_KV_HEADS) * p->desc.page_size * p->rb_k;
  info->v_page_bytes = static_cast<size_t>(PA_N_KV_HEADS) * p->desc.page_size * p->rb_v;
  info->n_blocks = p->desc.n_blocks;
  info->n_free = p->alloc.n_free();
  info->page_size = p->desc.page_size;
  info->kv_type = PA_KV_TYPE(p->k_type, p->v_type);
  info->max_blocks_per_seq = p->desc.max_blocks_per_seq;
  info->max_seqs = p->desc.max_seqs;
  info->device = p->desc.device;
  return PA_OK;
}

pa_status pa_alloc_blocks(pa_pool* p, int32_t n, pa_block* handles, int32_t* indices) {
  if (!p || n < 0) return PA_ERR_INVALID;
  if (n == 0) return PA_OK;
  if (!handles && !indices) return PA_ERR_INVALID;
  std::lock_guard<std::mutex> lk(p->mu);
  switch (p->alloc.alloc(n, handles, indices)) {
    case BlockAllocator::kOk: return PA_OK;
    case BlockAllocator::kNoMem: return PA_ERR_NOMEM;
    default: return PA_ERR_INVALID;
  }
}

pa_status pa_free_blocks(pa_pool* p, int32_t n, const pa_block* handles) {
  if (!p || n < 0 || (n > 0 && !handles)) return PA_ERR_INVALID;
  if (n == 0) return PA_OK;
  std::lock_guard<std::mutex> lk(p->mu);
  switch (p->alloc.free(n, handles)) {
    case BlockAllocator::kOk: return PA_OK;
    case BlockAllocator::kStale: return PA_ERR_STALE;
    default: return PA_ERR_INVALID;
  }
}

pa_status pa_append_kv(pa_pool* p, int32_t n_rows, const int32_t* dst_block, const int32_t* dst_slot,
                       const void* k_rows, const void* v_rows, hipStream_t stream) {
  if (!p || n_rows < 0) return PA_ERR_INVALID;
  if (n_rows == 0) return PA_OK;
  if (!dst_block || !dst_slot || !k_rows || !v_rows) return PA_ERR_INVALID;
  if (p->desc.flags & PA_POOL_HOST_ONLY) return PA_ERR_INVALID;
  std::lock_guard<std::mutex> lk(p->mu);
  const int P = p->desc.page_size;
  // Validate everything before enqueueing anything; keep only the last row of
  // each destination so that the later row wins whatever the kernel order.
  std::unordered_map<int64_t, int32_t> last;
  last.reserve(static_cast<size_t>(n_rows) * 2);
  for (int32_t i = 0; i < n_rows; ++i) {
    const int32_t b = dst_block[i], s = dst_slot[i];
    if (b < 0 || b >= p->desc.n_blocks || s < 0 || s >= P || !p->alloc.is_allocated(b)) return PA_ERR_INVALID;
    last[static_cast<int64_t>(b) * P + s] = i;
  }
  std::vector<int32_t> order;
  order.reserve(last.size());
  for (int32_t i = 0; i < n_rows; ++i)
    if (last[static_cast<int64_t>(dst_block[i]) * P + dst_slot[i]] == i) order.push_back(i);

  DeviceGuard dg(p->desc.device);
  if (!dg.ok) return PA_ERR_HIP;
  const size_t krow = static_cast<size_t>(PA_N_KV_HEADS) * p->rb_k;
  const size_t vrow = static_cast<size_t>(PA_N_KV_HEADS) * p->rb_v;
  const int cap = p->desc.max_append_rows;
  for (size_t first = 0; first < order.size(); first += cap) {
    const int n = static_cast<int>(std::min(order.size() - first, static_cast<size_t>(cap)));
    Staging& sl = p->staging[p->next_slot];
    p->next_slot = (p->next_slot + 1) % kStagingSlots;
    if (sl.used) {
      const hipError_t e = hipEventSynchronize(sl.done);   // the slot's previous batch has been consumed
      if (e != hipSuccess) return hip_status(e);
    }
    uint8_t* h = static_cast<uint8_t*>(sl.host);
    int32_t* hb = reinterpret_cast<int32_t*>(h);
    const size_t koff = pa::staging_k_off(n), voff = pa::staging_v_off(n, p->rb_k);
    for (int r = 0; r < n; ++r) {
      const int32_t i = order[first + r];
      hb[r] = dst_block[i];
      hb[n + r] = dst_slot[i];
      std::memcpy(h + koff + r * krow, static_cast<const uint8_t*>(k_rows) + i * krow, krow);
      std::memcpy(h + voff + r * vrow, static_cast<const uint8_t*>(v_rows) + i * vrow, vrow);
    }
    // The upload runs on the pool's own copy stream, so that it overlaps work
    // already enqueued on `stream` (the previous decode); `stream` waits for
    // it before the scatter.  The slot's previous scatter has finished (the
    // wait above), so nothing still reads its device staging.
    const size_t bytes = pa::staging_bytes(n, p->rb_k, p->rb_v);
    hipError_t e = hipMemcpyAsync(sl.dev, sl.host, bytes, hipMemcpyHostToDevice, p->copy_stream);
    if (e == hipSuccess) e = hipEventRecord(sl.copied, p->copy_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, sl.copied, 0);
    if (e == hipSuccess)
      e = pa::launch_scatter(static_cast<const uint8_t*>(sl.dev), n, static_cast<uint8_t*>(p->desc.k_pool),
                             static_cast<uint8_t*>(p->desc.v_pool), p->rb_k, p->rb_v, P, stream);
    if (e == hipSuccess) e = hipEventRecord(sl.done, stream);
    if (e != hipSuccess) return hip_status(e);
    sl.used = true;
  }
  return PA_OK;
}

pa_status pa_append_kv_device(pa_pool* p, int32_t n_rows, const int32_t* dst_block, const int32_t* dst_slot,
                              const void* k_src, const void* v_src, int32_t src_type, int32_t* err_word,
                              hipStream_t stream) {
  if (!p || n_rows < 0) return PA_ERR_INVALID;
  if (src_type != PA_F32 && src_type != PA_BF16 && src_type != PA_F16) return PA_ERR_INVALID;
  if (n_rows == 0) return PA_OK;
  if (!dst_block || !dst_slot || !k_src || !v_src) return PA_ERR_INVALID;
  if (p->desc.flags & PA_POOL_HOST_ONLY) return PA_ERR_INVALID;
  if (!aligned(k_src, 16) || !aligned(v_src, 16) || !aligned(dst_block, 4) || !aligned(dst_slot, 4) ||
      (err_word && !aligned(err_word, 4)))
    return PA_ERR_INVALID;
  uint32_t* err = err_word ? reinterpret_cast<uint32_t*>(err_word) : static_cast<uint32_t*>(p->workspace);
  if (!err) return PA_ERR_INVALID;
  DeviceGuard dg(p->desc.device);
  if (!dg.ok) return PA_ERR_HIP;
  pa::AppendLaunch l;
  l.k_src = k_src;
  l.v_src = v_src;
  l.src_type = src_type;
  l.k_pool = static_cast<uint8_t*>(p->desc.k_pool);
  l.v_pool = static_cast<uint8_t*>(p->desc.v_pool);
  l.k_type = p->k_type;
  l.v_type = p->v_type;
  l.dst_block = dst_block;
  l.dst_slot = dst_slot;
  l.err = err;
  l.n_rows = n_rows;
  l.n_blocks = p->desc.n_blocks;
  l.page_size = p->desc.page_size;
  return hip_status(pa::launch_append_encode(l, stream));
}

namespace {

constexpr int kGroupTokens = 8;   // query tokens of one prefill row tile

int n_groups_of(int n_qtok) { return (n_qtok + kGroupTokens - 1) / kGroupTokens; }

// Item target the workspace of a call is sized for: decode, the whole
// target; prefill, the target shared among the token groups.
int64_t sizing_target(int n_qtok, bool prefill, int device) {
  const int64_t t = target_items(device);
  if (!prefill) return t;
  const int64_t g = n_groups_of(n_qtok);
  return (t + g - 1) / g;
}

// Work items (of 6 n_qtok partial rows for decode, 48 for prefill) the
// workspace must hold.
int64_t workspace_items(int64_t n_seq, int n_qtok, bool prefill, int device) {
  const int64_t per_group = pa::max_work_items(n_seq, sizing_target(n_qtok, prefill, device));
  return prefill ? per_group * n_groups_of(n_qtok) : per_group;
}

int workspace_rows_tokens(int n_qtok, bool prefill) { return prefill ? kGroupTokens : n_qtok; }

// Item target, grid bound and one-round budget of the chunk plan for
// `slots` resident split workgroups, with `cap_target` the target the
// workspace was sized for.
struct PlanParams {
  int64_t target, max_items, budget, split, slots;
};
PlanParams plan_params(int64_t n_seq, int64_t slots, int64_t cap_target) {
  PlanParams r;
  r.slots = slots;
  r.target = pa::plan_target(n_seq, slots, cap_target);
  r.split = pa::split_target(n_seq, slots, cap_target);
  // the grid covers the items of either target
  r.max_items = pa::max_work_items(n_seq, r.split > r.target ? r.split : r.target);
  // when every item fits one round, the plan may shorten the chunk as long
  // as the items stay within the grid (max_items)
  r.budget = (2 * static_cast<int64_t>(pa::kKvHeads) * n_seq <= slots) ? r.max_items : 0;
  return r;
}

// Decode and prefill: one implementation, the query tokens taken in groups
// (one token group per workgroup; see group_tok below).
pa_status attend(const float* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                 const int32_t* seq_lens, int32_t n_seq, int32_t n_qtok, int32_t kv_type, int32_t page_size,
                 float* out, hipStream_t stream, const pa_decode_ext* ext, bool prefill) {
  const int max_tok = prefill ? PA_MAX_PREFILL_TOKENS : PA_MAX_QTOK;
  if (n_seq < 0 || n_qtok < 1 || n_qtok > max_tok) return PA_ERR_INVALID;
  int kt = 0, vt = 0;
  const pa_status ts = parse_kv_type(kv_type, &kt, &vt);
  if (ts != PA_OK) return ts;
  if (!page_size_ok(page_size)) return PA_ERR_UNSUPPORTED;
  if (!k_pool || !v_pool) return PA_ERR_INVALID;
  if (n_seq == 0) return PA_OK;
  if (!q || !out || !seq_lens) return PA_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(seq_lens, 4) || (block_table && !aligned(block_table, 4)))
    return PA_ERR_INVALID;

  int device = 0;
  int32_t bt_stride = 0, n_pool_blocks = 0;
  float scale = 0.f;
  float* lse_out = nullptr;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  const int32_t* lens_host = nullptr;
  int engine = 0;
  if (ext) {
    engine = (ext->flags & PA_DECODE_VECTOR_REFERENCE) ? 1 : 0;
    if ((ext->flags & ~PA_DECODE_VECTOR_REFERENCE) || ext->bt_stride < 1) return PA_ERR_INVALID;
    if (block_table && ext->n_pool_blocks < 1) return PA_ERR_INVALID;
    if (ext->lse_out && !aligned(ext->lse_out, 4)) return PA_ERR_INVALID;
    if (!std::isfinite(ext->scale)) return PA_ERR_INVALID;
    bt_stride = ext->bt_stride;
    n_pool_blocks = ext->n_pool_blocks;
    scale = ext->scale;
    lse_out = ext->lse_out;
    ws = ext->workspace;
    ws_bytes = ext->workspace_bytes;
    ev0 = static_cast<hipEvent_t>(ext->split_events[0]);
    ev1 = static_cast<hipEvent_t>(ext->split_events[1]);
    lens_host = ext->seq_lens_host;
    // Without a usable device the launch below reports the HIP error; the
    // remaining host checks still run first.
    if (hipGetDevice(&device) != hipSuccess) device = 0;
  }
  pa_pool* pool = nullptr;
  if (!ext || !ws) {
    std::lock_guard<std::mutex> lk(g_registry_mu);
    auto it = g_registry.find(k_pool);
    if (it == g_registry.end()) return ext ? PA_ERR_INVALID : PA_ERR_NOT_FOUND;
    pool = it->second;
  }
  if (pool) {
    if (pool->desc.v_pool != v_pool || pool->desc.page_size != page_size ||
        PA_KV_TYPE(pool->k_type, pool->v_type) != PA_KV_TYPE(kt, vt))
      return PA_ERR_INVALID;
    if (!ext) {
      if (!block_table) return PA_ERR_INVALID;
      bt_stride = pool->desc.max_blocks_per_seq;
      n_pool_blocks = pool->desc.n_blocks;
      device = pool->desc.device;
    }
    if (!ws) {
      if (n_seq > pool->desc.max_seqs) return PA_ERR_INVALID;
      ws = pool->workspace;
      ws_bytes = pool->workspace_bytes;
      device = pool->desc.device;
    }
  }
  if (static_cast<int64_t>(bt_stride) * page_size > (1ll << 30)) return PA_ERR_INVALID;
  const int64_t target = sizing_target(n_qtok, prefill, device);
  if (!ws || !aligned(ws, 256)) return PA_ERR_INVALID;
  const pa::WorkspaceLayout wl = pa::workspace_layout_for_bytes(ws_bytes, workspace_rows_tokens(n_qtok, prefill));
  const int64_t items = workspace_items(n_seq, n_qtok, prefill, device);
  if (wl.items < items) return PA_ERR_INVALID;

  pa::DecodeParams prm{};
  prm.q = q;
  prm.k = static_cast<const uint8_t*>(k_pool);
  prm.v = static_cast<const uint8_t*>(v_pool);
  prm.bt = block_table;
  prm.seq_lens = seq_lens;
  prm.out = out;
  prm.lse_out = lse_out;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  prm.err = reinterpret_cast<uint32_t*>(wsb);
  prm.part_lse = reinterpret_cast<float*>(wsb + wl.lse_off);
  prm.part_o = reinterpret_cast<float*>(wsb + wl.o_off);
  prm.n_seq = n_seq;
  prm.n_qtok = n_qtok;
  prm.bt_stride = bt_stride;
  prm.page_size = page_size;
  prm.page_shift = ((page_size & (page_size - 1)) == 0) ? __builtin_ctz(static_cast<unsigned>(page_size)) : -1;
  prm.n_pool_blocks = block_table ? n_pool_blocks : 0;
  // The plan aims at one round of resident workgroups (shared among the
  // token groups of a prefill); the workspace check above used the larger
  // capacity target, so these items always fit.
  // Tokens per split launch group.  On the matrix-core path a kernel holds
  // at most four tokens' output tiles from six tokens up, so two workgroups
  // fit a compute unit: decode keeps up to five tokens in one group and
  // halves six to eight (seven: a group of four and one of three in the
  // four-token kernel), prefill takes groups of four, the last possibly
  // partial.  The vector path takes decode whole and prefill in groups of
  // eight.  `groups` of them share one launch's grid (the vector path runs a
  // partial last group in a launch of its own).
  int group_tok = prefill ? (engine == 0 ? 4 : kGroupTokens)
                          : ((engine == 0 && n_qtok >= 6) ? (n_qtok + 1) / 2 : n_qtok);
  if (group_tok > n_qtok) group_tok = n_qtok;
  const int groups = (n_qtok + group_tok - 1) / group_tok;
  const int kernel_tok = n_qtok < group_tok ? n_qtok : group_tok;
  const int cu = cu_count(device);
  const int64_t slots = static_cast<int64_t>(cu > 0 ? cu : 256) * pa::split_wgs_per_cu(kt, vt, kernel_tok, engine);
  const int64_t per_group_slots = slots / groups > 0 ? slots / groups : 1;
  const PlanParams pp = plan_params(n_seq, per_group_slots, target);
  // A dispatch holds at most 2^32 - 1 work items: both grids (split: the
  // plan's items per token group times the groups; merge: one workgroup per
  // query row at most) must fit before anything is enqueued.
  const int64_t max_wgs = ((1ll << 32) - 1) / 256;
  const int64_t items_padded = groups > 1 ? (pp.max_items + 7) / 8 * 8 : pp.max_items;   // blocks of 8 with groups
  if (items_padded * groups > max_wgs || static_cast<int64_t>(n_seq) * PA_N_Q_HEADS * n_qtok > max_wgs)
    return PA_ERR_UNSUPPORTED;
  prm.target_items = static_cast<int32_t>(pp.target);
  prm.max_items = static_cast<int32_t>(pp.max_items);
  prm.plan_budget = static_cast<int32_t>(pp.budget);
  prm.split_target = static_cast<int32_t>(pp.split);
  prm.plan_slots = static_cast<int32_t>(pp.slots);
  prm.n_cu = cu > 0 ? cu : 256;
  prm.tok_total = n_qtok;
  prm.tok0 = 0;
  prm.n_groups = 1;
  prm.group_tok = group_tok;
  prm.part_rows = 6 * workspace_rows_tokens(n_qtok, prefill);
  prm.part_items = prm.max_items;
  prm.k_type = kt;
  prm.v_type = vt;
  prm.engine = engine;
  const float sc = (scale == 0.f) ? 1.0f / 16.0f : scale;
  prm.scale_log2 = sc * 1.4426950408889634f;
  prm.hp.on = 0;
  if (lens_host && n_seq <= pa::kHostPlanSeqs)
    pa::host_plan(lens_host, n_seq, bt_stride * page_size, prm.target_items, prm.plan_budget, prm.split_target,
                  prm.plan_slots, n_qtok, prm.hp);
  return hip_status(pa::launch_decode(prm, stream, ev0, ev1));
}

}  // namespace

pa_status pa_decode(const float* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                    const int32_t* seq_lens, int32_t n_seq, int32_t n_qtok, int32_t kv_type, int32_t page_size,
                    float* out, hipStream_t stream, const pa_decode_ext* ext) {
  return attend(q, k_pool, v_pool, block_table, seq_lens, n_seq, n_qtok, kv_type, page_size, out, stream, ext,
                false);
}

pa_status pa_prefill(const float* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                     const int32_t* seq_lens, int32_t n_seq, int32_t n_qtok, int32_t kv_type, int32_t page_size,
                     float* out, hipStream_t stream, const pa_decode_ext* ext) {
  return attend(q, k_pool, v_pool, block_table, seq_lens, n_seq, n_qtok, kv_type, page_size, out, stream, ext,
                true);
}

pa_status pa_split_plan(const int32_t* seq_lens_host, int32_t n_seq, int32_t cap, int32_t n_cu, int32_t wgs_per_cu,
                        int32_t* chunk, int32_t* n_items, int32_t* first) {
  if (!chunk || !n_items || n_seq < 0 || n_seq > PA_HOST_PLAN_MAX_SEQS || cap < 1 || n_cu < 1 || wgs_per_cu < 1 ||
      (n_seq > 0 && !seq_lens_host))
    return PA_ERR_INVALID;
  if (n_seq == 0) {
    *chunk = 0;
    *n_items = 0;
    if (first) first[0] = 0;
    return PA_OK;
  }
  const PlanParams pp = plan_params(n_seq, static_cast<int64_t>(n_cu) * wgs_per_cu,
                                    static_cast<int64_t>(n_cu) * kTargetPerCu);
  pa::HostPlan hp;
  pa::host_plan(seq_lens_host, n_seq, cap, static_cast<int>(pp.target), static_cast<int>(pp.budget),
                static_cast<int>(pp.split), static_cast<int>(pp.slots), 1, hp);
  *chunk = hp.chunk;
  *n_items = pa::kKvHeads * hp.first[n_seq];
  if (first)
    for (int i = 0; i <= n_seq; ++i) first[i] = hp.first[i];
  return PA_OK;
}

pa_status pa_split_workgroups_per_cu(int32_t kv_type, int32_t n_qtok, uint32_t flags, int32_t* wgs) {
  if (!wgs || n_qtok < 1 || n_qtok > PA_MAX_QTOK || (flags & ~PA_DECODE_VECTOR_REFERENCE)) return PA_ERR_INVALID;
  int kt = 0, vt = 0;
  const pa_status ts = parse_kv_type(kv_type, &kt, &vt);
  if (ts != PA_OK) return ts;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return PA_ERR_HIP;
  *wgs = pa::split_wgs_per_cu(kt, vt, n_qtok, (flags & PA_DECODE_VECTOR_REFERENCE) ? 1 : 0);
  return PA_OK;
}

pa_status pa_prefill_workspace_size(int32_t n_seq, int32_t n_qtok, int32_t device, size_t* bytes) {
  if (!bytes || n_seq < 0 || n_qtok < 1 || n_qtok > PA_MAX_PREFILL_TOKENS) return PA_ERR_INVALID;
  *bytes = pa::workspace_layout_items(workspace_items(n_seq, n_qtok, true, device), kGroupTokens).total;
  return PA_OK;
}

pa_status pa_get_device_error(pa_pool* pool, void* workspace, hipStream_t stream, int32_t clear, int32_t* err) {
  if (!err) return PA_ERR_INVALID;
  void* ws = workspace;
  if (!ws && !pool) {                       // pa_decode_scratch's buffer on the current device
    pa_status st = PA_OK;
    ws = pa::scratch_buffer(&st);
    if (st != PA_OK) return st;
  }
  if (!ws) {
    if (!pool->workspace) return PA_ERR_INVALID;
    ws = pool->workspace;
  }
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e == hipSuccess && clear) e = hipMemsetAsync(ws, 0, sizeof(int32_t), stream);
  if (e != hipSuccess) return hip_status(e);
  *err = v;
  return PA_OK;
}

pa_status pa_read_bandwidth_probe_ex(const void* src, size_t bytes, uint32_t* sink, size_t sink_words,
                                     int32_t wgs_per_cu, int32_t loads_in_flight, uint32_t flags,
                                     hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || !aligned(src, 16) || !aligned(sink, 4)) return PA_ERR_INVALID;
  if (wgs_per_cu < 1 || wgs_per_cu > 32 || (flags & ~(PA_PROBE_SLICE | PA_PROBE_LDS))) return PA_ERR_INVALID;
  const int u = loads_in_flight;
  if (u != 1 && u != 2 && u != 4 && u != 8 && u != 16) return PA_ERR_INVALID;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) device = 0;
  const int cu = cu_count(device);
  const int64_t blocks = static_cast<int64_t>(cu > 0 ? cu : 256) * wgs_per_cu;
  if (static_cast<int64_t>(sink_words) < blocks * 4) return PA_ERR_INVALID;
  return hip_status(pa::launch_read_probe(src, bytes, sink, static_cast<int32_t>(blocks), u,
                                          (flags & PA_PROBE_LDS) != 0, (flags & PA_PROBE_SLICE) != 0, stream));
}

pa_status pa_read_bandwidth_probe(const void* src, size_t bytes, uint32_t* sink, size_t sink_words,
                                  hipStream_t stream) {
  return pa_read_bandwidth_probe_ex(src, bytes, sink, sink_words, PA_PROBE_DEFAULT_WGS, PA_PROBE_DEFAULT_LOADS,
                                    PA_PROBE_DEFAULT_FLAGS, stream);
}

pa_status pa_debug_gather(const void* pool, int32_t row_bytes, const int32_t* block_table, int32_t bt_stride,
                          int32_t n_pool_blocks, int32_t seq, int32_t seq_len, int32_t page_size, void* dst,
                          int32_t* err_word, hipStream_t stream) {
  if (!pool || !dst || seq < 0 || seq_len < 0 || bt_stride < 1 || row_bytes <= 0 || row_bytes % 16) return PA_ERR_INVALID;
  if (!page_size_ok(page_size)) return PA_ERR_UNSUPPORTED;
  if (block_table && n_pool_blocks < 1) return PA_ERR_INVALID;
  if (static_cast<int64_t>(seq_len) > static_cast<int64_t>(bt_stride) * page_size) return PA_ERR_INVALID;
  if (!aligned(pool, 16) || !aligned(dst, 16)) return PA_ERR_INVALID;
  return hip_status(pa::launch_gather(static_cast<const uint8_t*>(pool), row_bytes, block_table, bt_stride,
                                      n_pool_blocks, seq, seq_len, page_size, static_cast<uint8_t*>(dst), err_word,
                                      stream));
}

}  // extern "C"
