// Internal interface between the C ABI (pa_host.cpp) and the kernels
// (pa_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#define PA_HD __host__ __device__

namespace pa {

constexpr int kHeadDim = 256;
constexpr int kQHeads = 24;
constexpr int kKvHeads = 4;
constexpr int kGroup = kQHeads / kKvHeads;  // query heads per KV head
constexpr int kMaxQtok = 8;
constexpr int kChunkGranule = 128;          // chunk lengths are multiples of this (32 keys x 4 waves)
constexpr int kPlanCand = 4;                // chunk lengths the plan tries at once
constexpr int kMaxWaves = 8;                // waves of the largest workgroup
constexpr int kPlanShared = kMaxWaves * kPlanCand;  // long long slots of the plan's shared scratch

enum KvType { kF16 = 1, kBF16 = 2, kQ8_0 = 3, kQ4_0 = 4 };

// Value types of the source rows of a device-side append (PA_F32, PA_BF16,
// PA_F16).
enum SrcType { kSrcF16 = 1, kSrcBF16 = 2, kSrcF32 = 5 };

inline int row_bytes_of(int t) {
  switch (t) {
    case kF16: case kBF16: return 512;
    case kQ8_0: return 8 * 34;
    case kQ4_0: return 8 * 18;
    default: return 0;
  }
}

// Merge of chunk partials: chunk outputs per lane in flight, and the
// workgroups the compact merge grid gives a sequence of nc chunks and `rows`
// query rows (a row of up to kMergeBatch chunks is merged by one wave, four
// rows per workgroup; a longer row by a workgroup; one chunk needs none).
constexpr int kMergeBatch = 32;
PA_HD inline int merge_wgs(int nc, int rows) {
  if (nc <= 1) return 0;
  return nc > kMergeBatch ? rows : (rows + 3) / 4;
}

// The chunk plan computed on the host from a host copy of seq_lens (up to
// kHostPlanSeqs sequences), carried in the launch arguments: the kernels then
// locate their work item without reading seq_lens.  Same integer arithmetic
// as the device plan (plan_wg), so both give the same chunks.
constexpr int kHostPlanSeqs = 256;
struct HostPlan {
  int32_t on;                       // 1: the fields below hold the plan
  int32_t chunk;                    // chunk length in positions
  int32_t any_multi;                // some sequence has more than one chunk (the merge has work)
  int32_t first[kHostPlanSeqs + 1]; // plan index of sequence s's first chunk; first[n_seq] = all pairs
  int32_t len[kHostPlanSeqs];       // seq_lens
  int32_t mfirst[kHostPlanSeqs + 1];// first merge workgroup of sequence s; mfirst[n_seq] = the merge grid
  // Longest-first order of a grid of several rounds (lpt = 1): the split
  // workgroups take every full-length chunk first (in plan order), then the
  // shorter last chunks by decreasing length, so the last round holds the
  // shortest work.  pmask bit s: sequence s ends in a chunk shorter than
  // `chunk` (or is empty); n_full: chunks of full length; ord: the sequences
  // with a short last chunk, longest first.  Results do not depend on it.
  int32_t lpt;
  int32_t n_full;
  uint32_t pmask[kHostPlanSeqs / 32];
  uint8_t ord[kHostPlanSeqs];
};

// Everything one decode launch needs.  Device pointers unless noted.
struct DecodeParams {
  const float* q;          // [n_seq][n_qtok][24][256]
  const uint8_t* k;        // pool or contiguous storage
  const uint8_t* v;
  const int32_t* bt;       // [n_seq][bt_stride], or nullptr (contiguous)
  const int32_t* seq_lens; // [n_seq]
  float* out;              // [n_seq][n_qtok][24][256]
  float* lse_out;          // [n_seq][n_qtok][24] or nullptr
  float* part_o;           // [item capacity][24][256]
  float* part_lse;         // [item capacity][24]   (log2 units)
  uint32_t* err;           // error word
  int32_t n_seq, n_qtok, bt_stride, page_size, n_pool_blocks;
  int32_t page_shift;      // log2(page_size) when it is a power of two, else -1
  int32_t target_items;    // item target of the chunk plan (plan_target)
  int32_t plan_budget;     // > 0: the plan takes the shortest chunk whose items fit in it
  int32_t split_target;    // > 0: the target of a ragged many-sequence batch (split_target)
  int32_t plan_slots;      // co-resident split workgroups (for ragged_split)
  int32_t n_cu;            // compute units: the first n_cu workgroups of a grid land one per unit
  int32_t max_items;       // work items of the plan the grid covers (per token group)
  // Token groups: q / out / lse_out hold tok_total tokens per sequence,
  // taken group_tok at a time.  On the matrix-core path every group runs
  // in one launch (n_groups of them from token tok0, in a grid of max_items
  // x n_groups workgroups, max_items rounded up to 8 when there are several
  // groups, whose groups of one item sit 8 workgroups apart on one XCD), a
  // partial last group masking its missing tokens; decode takes up to five
  // tokens in one group and six to eight in two, prefill groups of four (so
  // no kernel holds more than four tokens' output tiles from six tokens up).
  // The vector path takes decode whole and prefill in groups of eight, the
  // full groups in one launch and the rest in a second.
  int32_t tok_total, tok0, n_groups, group_tok;
  // Chunk partials of the tokens 8g.. 8g+7 and plan item i start at row
  // (g * part_items + i) * part_rows of part_o / part_lse; token t's six
  // rows sit 6 (t % 8) rows in.
  int32_t part_rows, part_items;
  int32_t k_type, v_type;
  int32_t engine;          // 0: matrix-core path, 1: fp32 vector reference path
  float scale_log2;        // softmax scale * log2(e)
  HostPlan hp;             // hp.on == 0: the kernels compute the plan from seq_lens
};

// Upper bound on work items for n_seq sequences (see the plan in the kernels).
inline int64_t max_work_items(int64_t n_seq, int64_t target_items) {
  return target_items + kKvHeads * n_seq;
}

// Item target of the chunk plan for `slots` co-resident workgroups.  The plan
// yields at most target + 4 n_seq items, so when the sequences leave room the
// target fills exactly one round of resident workgroups (no second wave of
// short-lived workgroups, each paying the set-up again); otherwise half a
// round of chunks goes on top of the one-item-per-(sequence, head) minimum.
// Never above `cap`, the target the workspace was sized for.
inline int64_t plan_target(int64_t n_seq, int64_t slots, int64_t cap) {
  const int64_t per = kKvHeads * n_seq;
  int64_t t = (2 * per <= slots) ? slots - per : slots / 2;
  if (t < 1) t = 1;
  return t < cap ? t : cap;
}

// The target a many-sequence batch switches to when it is ragged (0 when the
// sequences leave room for one round): two rounds of chunks of half a slot's
// share, which the hardware dispatcher spreads over the compute units as they
// free up.  The plan takes it when the longest valid sequence exceeds 1.5
// times a slot's share of the work, 4 sum(L) / slots (ragged_split); a batch
// of even lengths keeps one chunk per (sequence, head), which already
// balances.
inline int64_t split_target(int64_t n_seq, int64_t slots, int64_t cap) {
  const int64_t per = kKvHeads * n_seq;
  if (2 * per <= slots) return 0;
  const int64_t t = 2 * slots;
  return t < cap ? t : cap;
}

PA_HD inline bool ragged_split(long long max_len, long long total, long long slots) {
  return 2 * max_len * slots > 3 * static_cast<long long>(kKvHeads) * total;
}

// Work items the split grid covers (per token group): the plan's exact count
// with a host plan, else the bound max_items.
inline int32_t grid_items(const DecodeParams& p) {
  return p.hp.on ? kKvHeads * p.hp.first[p.n_seq] : p.max_items;
}

// Fills `hp` from host seq_lens (n_seq <= kHostPlanSeqs) with the device
// plan's arithmetic for the given target and budget; the merge grid is laid
// out for tok_total query tokens per sequence.
void host_plan(const int32_t* lens, int n_seq, int cap, int target, int budget, int split, int slots, int tok_total,
               HostPlan& hp);

// Resident workgroups per compute unit of the split kernel a call selects
// (from the runtime's occupancy query; at least 1).
int split_wgs_per_cu(int k_type, int v_type, int n_qtok, int engine);

struct WorkspaceLayout {
  int64_t items;       // work-item capacity
  size_t lse_off, o_off, total;
};

PA_HD inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Partial rows of one work item: the 6 query heads x n_qtok tokens.
PA_HD constexpr int rows_per_item(int n_qtok) { return 6 * n_qtok; }

// The workspace header's int32 words: [0] the device error word, [1] the
// call's chunk length and [2 + s] the plan index of sequence s's first chunk
// for s < kHdrSeqs, written by the split kernel for the merge kernel (larger
// batches make the merge compute the plan again).
constexpr int kHdrBytes = 4096;
constexpr int kHdrSeqs = kHdrBytes / 4 - 2;

// Workspace: [0, kHdrBytes) header (error word at 0); chunk log-sum-exps
// [items][6 n_qtok]; chunk outputs [items][6 n_qtok][256].  The layout
// depends on the call's n_qtok and the item capacity only, so a workspace
// sized for n_qtok tokens also serves every call of fewer tokens (more items
// fit).  The error word must be zero before the first call.
inline WorkspaceLayout workspace_layout_items(int64_t items, int n_qtok) {
  const size_t rows = static_cast<size_t>(rows_per_item(n_qtok));
  WorkspaceLayout w;
  w.items = items;
  w.lse_off = kHdrBytes;
  w.o_off = align_up(w.lse_off + static_cast<size_t>(items) * rows * sizeof(float), 256);
  w.total = align_up(w.o_off + static_cast<size_t>(items) * rows * kHeadDim * sizeof(float), 256);
  return w;
}

inline WorkspaceLayout workspace_layout(int64_t n_seq, int64_t target_items, int n_qtok) {
  return workspace_layout_items(max_work_items(n_seq, target_items), n_qtok);
}

// The largest item capacity whose layout for n_qtok tokens fits in `bytes`.
inline WorkspaceLayout workspace_layout_for_bytes(size_t bytes, int n_qtok) {
  const size_t per = rows_per_item(n_qtok) * sizeof(float) * (1 + kHeadDim);
  int64_t items = static_cast<int64_t>(bytes / per) + 1;   // an upper bound; step down to the largest fit
  while (items > 0 && workspace_layout_items(items, n_qtok).total > bytes) --items;
  return workspace_layout_items(items, n_qtok);
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_begin,
                         hipEvent_t ev_end);

// Where a split kernel is launched: the stream, and optional timing events
// that the runtime attaches to the dispatch itself (start: the kernel begins
// executing; stop: it has completed), so their interval is the kernel's run
// time, not the time between two marker packets around it.
struct SplitLaunch {
  hipStream_t stream;
  hipEvent_t start;
  hipEvent_t stop;
};

// Split kernels for n_qtok = T: each T is its own translation unit (the
// matrix-core and vector sources are built once per T with -DPA_T=T), so
// the instantiations of all K x V encodings compile in parallel.
template <int T> hipError_t launch_split_mfma_t(const DecodeParams& p, const SplitLaunch& l);
template <int T> int split_mfma_wgs_t(int k_type, int v_type);
template <int T> hipError_t launch_split_valu_t(const DecodeParams& p, const SplitLaunch& l);
#define PA_DECLARE_SPLIT_T(T)                                                              \
  template <> hipError_t launch_split_mfma_t<T>(const DecodeParams& p, const SplitLaunch& l); \
  template <> int split_mfma_wgs_t<T>(int k_type, int v_type);                               \
  template <> hipError_t launch_split_valu_t<T>(const DecodeParams& p, const SplitLaunch& l);
PA_DECLARE_SPLIT_T(1)
PA_DECLARE_SPLIT_T(2)
PA_DECLARE_SPLIT_T(3)
PA_DECLARE_SPLIT_T(4)
PA_DECLARE_SPLIT_T(5)
PA_DECLARE_SPLIT_T(6)
PA_DECLARE_SPLIT_T(7)
PA_DECLARE_SPLIT_T(8)
#undef PA_DECLARE_SPLIT_T

// Staging layout for append: int32 block[n], int32 slot[n], then (16-byte
// aligned) K rows [n][4][rb_k], then V rows [n][4][rb_v].
PA_HD inline size_t staging_k_off(int64_t n) { return align_up(static_cast<size_t>(8 * n), 16); }
PA_HD inline size_t staging_v_off(int64_t n, int rb_k) { return staging_k_off(n) + static_cast<size_t>(n) * kKvHeads * rb_k; }
PA_HD inline size_t staging_bytes(int64_t n, int rb_k, int rb_v) {
  return staging_v_off(n, rb_k) + static_cast<size_t>(n) * kKvHeads * rb_v;
}

hipError_t launch_scatter(const uint8_t* staging, int32_t n_rows, uint8_t* k_pool, uint8_t* v_pool,
                          int32_t rb_k, int32_t rb_v, int32_t page_size, hipStream_t stream);

// Device-side append with fused encoding: rows [n_rows][4][256] of src_type
// values, encoded into the K and V pools' encodings and written at
// (dst_block[i], dst_slot[i]).  All pointers are device pointers.
struct AppendLaunch {
  const void* k_src;
  const void* v_src;
  int32_t src_type;
  uint8_t* k_pool;
  uint8_t* v_pool;
  int32_t k_type, v_type;
  const int32_t* dst_block;
  const int32_t* dst_slot;
  uint32_t* err;            // PA_DEVERR_APPEND is ORed in for a skipped row
  int32_t n_rows, n_blocks, page_size;
};

hipError_t launch_append_encode(const AppendLaunch& l, hipStream_t stream);

// Read-bandwidth probe: `blocks` workgroups read `bytes` (a multiple of 16)
// once with `unroll` (1, 2, 4, 8 or 16) 16-byte loads in flight per lane,
// into registers or straight to LDS, grid-stride or one contiguous slice per
// workgroup; sink receives blocks * 4 words.
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, int32_t unroll,
                             bool to_lds, bool slice, hipStream_t stream);

// The device address of pa_decode_scratch's buffer on the current device
// (taken once per device), or nullptr with *st set.
void* scratch_buffer(int32_t* st);

hipError_t launch_gather(const uint8_t* pool, int32_t row_bytes, const int32_t* bt, int32_t bt_stride,
                         int32_t n_pool_blocks, int32_t seq, int32_t seq_len, int32_t page_size,
                         uint8_t* dst, int32_t* err_word, hipStream_t stream);

}  // namespace pa
