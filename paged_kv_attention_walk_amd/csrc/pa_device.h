// Device helpers shared by the decode kernels: the row-address helper, the
// chunk plan, wave reductions, row decoding and the merge of chunk partials.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_internal.h"

namespace pa {
namespace dev {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.693147180559945309417f;
constexpr int kThreads = 256;
constexpr uint32_t kErrTable = 1u;
constexpr uint32_t kErrLength = 2u;

// -------------------------------------------------------------- row address
//
// The one row-address helper (ashhart/TensorFold issue 1156, Design /
// Kernels): with a table, position pos of sequence s lives in pool page
// bt[s][pos / P] at slot pos % P, and the pool is [page][KV head][slot][row];
// without a table, storage is [sequence][KV head][cap][row].  Returns a row
// index (multiply by the row size of K or V).  An entry outside the pool
// sets ok = false and yields row 0 of page 0, which is always in bounds.
__device__ inline size_t kv_row(const int32_t* __restrict__ bt, int bt_stride, int n_pool_blocks,
                                int page_size, int s, int h, int pos, bool& ok) {
  if (bt == nullptr) {
    ok = true;
    const size_t cap = static_cast<size_t>(bt_stride) * page_size;
    return (static_cast<size_t>(s) * kKvHeads + h) * cap + pos;
  }
  const int lp = pos / page_size;
  const int slot = pos - lp * page_size;
  int phys = bt[static_cast<size_t>(s) * bt_stride + lp];
  ok = static_cast<unsigned>(phys) < static_cast<unsigned>(n_pool_blocks);
  if (!ok) return 0;
  return (static_cast<size_t>(phys) * kKvHeads + h) * page_size + slot;
}

// --------------------------------------------------------------- the plan

__device__ inline bool len_ok(int L, int cap) { return L >= 0 && L <= cap; }

__device__ inline int n_chunks_of(int L, int cap, int chunk) {
  if (!len_ok(L, cap) || L == 0) return 1;
  return (L + chunk - 1) / chunk;
}

__device__ inline int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Waves of the calling workgroup (a multiple of 64 threads, at most
// kMaxWaves waves); the block-wide helpers below work for any such size.
__device__ inline int block_waves() { return static_cast<int>(blockDim.x) >> 6; }

// Block-wide sum of a per-thread value.  `sh` holds kMaxWaves slots.
__device__ inline long long block_sum(long long v, long long* sh) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  long long t = 0;
  for (int w = 0; w < block_waves(); ++w) t += sh[w];
  return t;
}

// Block-wide sums of kPlanCand per-thread values; `sh` holds kPlanShared
// slots.
__device__ inline void block_sum_vec(long long (&v)[kPlanCand], long long* sh) {
#pragma unroll
  for (int k = 0; k < kPlanCand; ++k)
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v[k] += __shfl_xor(v[k], d, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int k = 0; k < kPlanCand; ++k) sh[(threadIdx.x >> 6) * kPlanCand + k] = v[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kPlanCand; ++k) {
    long long t = 0;
    for (int w = 0; w < block_waves(); ++w) t += sh[w * kPlanCand + k];
    v[k] = t;
  }
}

// Block-wide maximum of a non-negative per-thread value.  `sh` holds
// kMaxWaves slots.
__device__ inline long long block_max(long long v, long long* sh) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const long long o = __shfl_xor(v, d, 64);
    v = o > v ? o : v;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  long long m = sh[0];
  for (int w = 1; w < block_waves(); ++w) m = sh[w] > m ? sh[w] : m;
  return m;
}

__device__ inline long long round_granule(long long c) {
  c = (c + kChunkGranule - 1) / kChunkGranule * kChunkGranule;
  if (c < kChunkGranule) c = kChunkGranule;
  return c > (1ll << 30) ? (1ll << 30) : c;
}

// Tokens per chunk, a multiple of the granule (32 keys for each of the 4
// waves of a workgroup).  From `target`: the total live length times the
// KV-head count spread over target items, rounded up -- the items then number
// at most target + 4 n_seq.  With budget > 0 (all items fit in one round of
// resident workgroups): the shortest chunk among the kPlanCand lengths from
// the lower bound 4 sum(L) / budget up whose items fit in the budget, if one
// of them is shorter than the length from target.  Shorter chunks give each
// wave fewer tiles.  `sh` holds kPlanShared slots.
__device__ inline int plan_chunk(const int32_t* __restrict__ lens, int n_seq, int cap, int target, int budget,
                                 int split, int slots, long long* sh) {
  long long acc = 0, mx = 0;
  for (int i = threadIdx.x; i < n_seq; i += blockDim.x) {
    const int L = lens[i];
    if (L > 0 && L <= cap) {
      acc += L;
      mx = L > mx ? L : mx;
    }
  }
  const long long total = block_sum(acc, sh);
  if (split > 0 && ragged_split(block_max(mx, sh), total, slots)) target = split;
  const long long c = round_granule((total * kKvHeads + target - 1) / target);
  if (budget <= 0 || total == 0) return static_cast<int>(c);
  const long long c0 = round_granule((total * kKvHeads + budget - 1) / budget);
  if (c0 >= c) return static_cast<int>(c);
  long long cnt[kPlanCand];
#pragma unroll
  for (int k = 0; k < kPlanCand; ++k) cnt[k] = 0;
  for (int i = threadIdx.x; i < n_seq; i += blockDim.x) {
    const int L = lens[i];
#pragma unroll
    for (int k = 0; k < kPlanCand; ++k) cnt[k] += n_chunks_of(L, cap, static_cast<int>(c0) + kChunkGranule * k);
  }
  block_sum_vec(cnt, sh);
#pragma unroll
  for (int k = 0; k < kPlanCand; ++k) {
    const long long ck = c0 + kChunkGranule * k;
    if (ck < c && kKvHeads * cnt[k] <= budget) return static_cast<int>(ck);
  }
  return static_cast<int>(c);
}

// Finds (s, c) of the j-th (sequence, chunk) pair; s = -1 when j is past the
// last one.  Wave 0 scans the per-sequence chunk counts; the result is
// broadcast through `sh` (2 ints).
__device__ inline void plan_locate(const int32_t* __restrict__ lens, int n_seq, int cap, int chunk, int j,
                                   int* sh) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int base = 0, fs = -1, fc = 0;
    for (int s0 = 0; s0 < n_seq; s0 += 64) {
      const int s = s0 + lane;
      const int nc = s < n_seq ? n_chunks_of(lens[s], cap, chunk) : 0;
      const int inc = wave_incl_scan(nc);
      const int excl = inc - nc;
      const bool hit = nc > 0 && j >= base + excl && j < base + inc;
      const unsigned long long m = __ballot(hit);
      if (m) {
        const int src = __ffsll(static_cast<long long>(m)) - 1;
        fs = s0 + src;
        fc = j - base - __shfl(excl, src, 64);
        break;
      }
      base += __shfl(inc, 63, 64);
    }
    if (lane == 0) {
      sh[0] = fs;
      sh[1] = fc;
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------ wave helpers

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = fmaxf(x, __shfl_xor(x, d, 64));
  return x;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

// Orders this wave's LDS accesses: everything before is visible to every lane
// of the wave after it.  A wave's LDS operations complete in issue order; the
// fence keeps the compiler from moving accesses across it.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// ----------------------------------------------------------- row decoding

__device__ inline float half_bits(uint32_t u) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<unsigned short>(u & 0xFFFFu)));
}
__device__ inline float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Byte `i` of a little-endian word array (i known at compile time after
// unrolling).
__device__ inline uint32_t byte_at(const uint32_t* w, int i) { return (w[i >> 2] >> (8 * (i & 3))) & 0xFFu; }

// Dot products of one whole K row (this lane's key) with R query rows held in
// LDS (row-major, 256 floats each, already multiplied by scale * log2 e).
template <int KT, int R>
__device__ inline void qk_row(const uint8_t* __restrict__ row, const float* __restrict__ q, float (&s)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) s[r] = 0.f;
  if constexpr (KT == kF16 || KT == kBF16) {
#pragma unroll 1
    for (int b = 0; b < 8; ++b) {
      uint32_t w[16];
      const uint4* src = reinterpret_cast<const uint4*>(row + 64 * b);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = src[i];
        w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
      }
      float x[32];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (KT == kF16) {
          x[2 * i] = half_bits(w[i]);
          x[2 * i + 1] = half_bits(w[i] >> 16);
        } else {
          x[2 * i] = bf16_lo(w[i]);
          x[2 * i + 1] = bf16_hi(w[i]);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float4* qq = reinterpret_cast<const float4*>(q + r * kHeadDim + 32 * b);
        float acc = s[r];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 qv = qq[i];
          acc += x[4 * i] * qv.x + x[4 * i + 1] * qv.y + x[4 * i + 2] * qv.z + x[4 * i + 3] * qv.w;
        }
        s[r] = acc;
      }
    }
  } else {
    constexpr int RB = (KT == kQ8_0) ? 272 : 144;
    constexpr int BB = (KT == kQ8_0) ? 34 : 18;
    uint32_t w[RB / 4];
    const uint4* src = reinterpret_cast<const uint4*>(row);
#pragma unroll
    for (int i = 0; i < RB / 16; ++i) {
      const uint4 v = src[i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int o = BB * b;
      const float d = half_bits(byte_at(w, o) | (byte_at(w, o + 1) << 8));
      float x[32];
      if constexpr (KT == kQ8_0) {
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = static_cast<float>(static_cast<int8_t>(byte_at(w, o + 2 + i)));
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t cb = byte_at(w, o + 2 + i);
          x[i] = static_cast<float>(static_cast<int>(cb & 15u) - 8);
          x[i + 16] = static_cast<float>(static_cast<int>(cb >> 4) - 8);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float4* qq = reinterpret_cast<const float4*>(q + r * kHeadDim + 32 * b);
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 qv = qq[i];
          acc += x[4 * i] * qv.x + x[4 * i + 1] * qv.y + x[4 * i + 2] * qv.z + x[4 * i + 3] * qv.w;
        }
        s[r] += d * acc;   // block scale applied to the block's exact-code dot product
      }
    }
  }
}

// Values of dims [4*lane, 4*lane+4) of one V row.
template <int VT>
__device__ inline void v_dims4(const uint8_t* __restrict__ row, int lane, float (&x)[4]) {
  if constexpr (VT == kF16 || VT == kBF16) {
    const uint2 w = *reinterpret_cast<const uint2*>(row + 8 * lane);
    if constexpr (VT == kF16) {
      x[0] = half_bits(w.x); x[1] = half_bits(w.x >> 16); x[2] = half_bits(w.y); x[3] = half_bits(w.y >> 16);
    } else {
      x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    }
  } else if constexpr (VT == kQ8_0) {
    const int b = lane >> 3, e = (lane & 7) * 4;
    const uint8_t* blk = row + 34 * b;
    const float d = half_bits(*reinterpret_cast<const uint16_t*>(blk));
    const uint32_t c01 = *reinterpret_cast<const uint16_t*>(blk + 2 + e);
    const uint32_t c23 = *reinterpret_cast<const uint16_t*>(blk + 4 + e);
    x[0] = d * static_cast<float>(static_cast<int8_t>(c01 & 0xFFu));
    x[1] = d * static_cast<float>(static_cast<int8_t>(c01 >> 8));
    x[2] = d * static_cast<float>(static_cast<int8_t>(c23 & 0xFFu));
    x[3] = d * static_cast<float>(static_cast<int8_t>(c23 >> 8));
  } else {
    const int b = lane >> 3, e = (lane & 7) * 4;
    const uint8_t* blk = row + 18 * b;
    const float d = half_bits(*reinterpret_cast<const uint16_t*>(blk));
    const int j0 = e & 15;
    const uint32_t c = *reinterpret_cast<const uint16_t*>(blk + 2 + j0) |
                       (static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(blk + 4 + j0)) << 16);
    const int sh = (e >= 16) ? 4 : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = d * static_cast<float>(static_cast<int>((c >> (8 * i + sh)) & 15u) - 8);
  }
}

// ------------------------------------------------------------------ merge
//
// Chunks of one (sequence, KV head) are combined by a second kernel.  For a
// query row: M = max lse; all -inf gives 0 with lse -inf (llama.cpp pull 2,
// pd_combine fix: an all-masked row is 0, not 0/0); a NaN partial (corrupt
// table) gives NaN; otherwise out = sum_c w_c o_c / sum_c w_c with
// w_c = 2^(lse_c - M) (lse in base 2).  A lane holds 4 dims (float4 loads).
// A row of at most kMergeBatch chunks is merged by one wave: every chunk in
// flight at once, summed in chunk order.  A longer row takes a whole
// workgroup: wave w takes chunks c = w, w+4, ..., up to kMergeBatch at once
// (a running base across batches), and the 4 waves' states are combined in
// wave order.  Which of the two a row takes depends only on its chunk count,
// so the result is bitwise the same whatever the grid, and repeatable.  With
// the host's plan the grid is compact: a sequence of one-wave rows takes
// 4 rows per workgroup, a sequence of longer rows one row per workgroup, and
// sequences of one chunk none (hp.mfirst, the prefix of these counts);
// otherwise one workgroup per row.

struct MergeShared {
  float4 part[4][64];
  float ml[4][2];
  long long sum[kPlanShared];
  int ints[4];
};

// Number of (sequence, chunk) pairs before sequence s.
__device__ inline int plan_prefix(const int32_t* __restrict__ lens, int s, int cap, int chunk, long long* sh) {
  long long acc = 0;
  for (int i = threadIdx.x; i < s; i += blockDim.x) acc += n_chunks_of(lens[i], cap, chunk);
  return static_cast<int>(block_sum(acc, sh));
}

// The plan as one workgroup needs it: the chunk length, and either the
// (sequence, chunk) of work item j (j >= 0) or the number of (sequence,
// chunk) pairs before sequence s_pref (s_pref >= 0).  Up to 64 sequences,
// wave 0 computes everything with wave-level reductions and one barrier
// publishes it; the same integer arithmetic as plan_chunk / plan_locate /
// plan_prefix, which serve longer batches.  `sh` holds kPlanShared slots,
// `shi` 4 ints.
struct PlanWG {
  int chunk, s, c, prefix;
  int len;      // seq_lens[s] when the host plan supplied it, else -1
  int item;     // plan index of chunk c of s (where its partial rows go)
};

__device__ inline long long wave_sum_ll(long long v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

__device__ inline int wave_sum_i(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

__device__ inline PlanWG plan_wg(const int32_t* __restrict__ lens, int n_seq, int cap, int target, int budget,
                                 int split, int slots, int j, int s_pref, long long* sh, int* shi) {
  PlanWG r{0, -1, 0, 0, -1, -1};
  if (n_seq > 64) {
    r.chunk = plan_chunk(lens, n_seq, cap, target, budget, split, slots, sh);
    if (j >= 0) {
      plan_locate(lens, n_seq, cap, r.chunk, j, shi);
      r.s = shi[0];
      r.c = shi[1];
    }
    if (s_pref >= 0) r.prefix = plan_prefix(lens, s_pref, cap, r.chunk, sh);
    return r;
  }
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const bool has = lane < n_seq;
    const int L = has ? lens[lane] : 0;
    const long long total = wave_sum_ll((has && L > 0 && L <= cap) ? L : 0);
    if (split > 0) {
      int mx = (has && L > 0 && L <= cap) ? L : 0;
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) mx = max(mx, __shfl_xor(mx, d, 64));
      if (ragged_split(mx, total, slots)) target = split;
    }
    long long chunk = round_granule((total * kKvHeads + target - 1) / target);
    if (budget > 0 && total > 0) {
      const long long c0 = round_granule((total * kKvHeads + budget - 1) / budget);
      if (c0 < chunk) {
        int cnt[kPlanCand];
#pragma unroll
        for (int k = 0; k < kPlanCand; ++k)
          cnt[k] = wave_sum_i(has ? n_chunks_of(L, cap, static_cast<int>(c0) + kChunkGranule * k) : 0);
        long long pick = chunk;
#pragma unroll
        for (int k = kPlanCand - 1; k >= 0; --k) {
          const long long ck = c0 + kChunkGranule * k;
          if (ck < chunk && static_cast<long long>(kKvHeads) * cnt[k] <= budget) pick = ck;
        }
        chunk = pick;
      }
    }
    const int nc = has ? n_chunks_of(L, cap, static_cast<int>(chunk)) : 0;
    int fs = -1, fc = 0, pref = 0;
    if (j >= 0) {
      const int inc = wave_incl_scan(nc);
      const int excl = inc - nc;
      const bool hit = nc > 0 && j >= excl && j < inc;
      const unsigned long long m = __ballot(hit);
      if (m) {
        const int src = __ffsll(static_cast<long long>(m)) - 1;
        fs = src;
        fc = j - __shfl(excl, src, 64);
      }
    }
    if (s_pref >= 0) pref = wave_sum_i(lane < s_pref ? nc : 0);
    if (lane == 0) {
      shi[0] = static_cast<int>(chunk);
      shi[1] = fs;
      shi[2] = fc;
      shi[3] = pref;
    }
  }
  __syncthreads();
  r.chunk = shi[0];
  r.s = shi[1];
  r.c = shi[2];
  r.prefix = shi[3];
  return r;
}

// The plan as plan_wg gives it, taken from the launch arguments when the
// host computed it (no load, no barrier), else computed from seq_lens.
// Lookup in the host plan's tables (launch arguments, n <= kHostPlanSeqs
// entries): the last s in [0, n) with key[s] <= j, for a non-decreasing key
// with key[0] <= j, and key[s], a[s], b[s].  Every lane reads its entries of
// all three tables at once and a ballot counts the keys <= j: one round
// trip to the argument memory instead of a binary search's chain of
// dependent loads.  Called by whole waves.
struct HostHit {
  int s, key, a, b;
};

__device__ inline HostHit host_lookup(const int32_t* key, const int32_t* a, const int32_t* b, int n, int j) {
  constexpr int kR = kHostPlanSeqs / 64;
  const int lane = threadIdx.x & 63;
  int kv[kR], av[kR], bv[kR];
  // the reads do not wait for n: every table holds kHostPlanSeqs entries
#pragma unroll
  for (int k = 0; k < kR; ++k) {
    const int i = 64 * k + lane;
    kv[k] = key[i];
    av[k] = a[i];
    bv[k] = b[i];
  }
#pragma unroll
  for (int k = 0; k < kR; ++k) kv[k] = (64 * k + lane < n) ? kv[k] : 0x7FFFFFFF;
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < kR; ++k) cnt += __popcll(__ballot(kv[k] <= j));
  HostHit r{cnt - 1, 0, 0, 0};
  const int src = r.s & 63;
#pragma unroll
  for (int k = 0; k < kR; ++k) {
    if ((r.s >> 6) == k) {
      r.key = __builtin_amdgcn_readlane(kv[k], src);
      r.a = __builtin_amdgcn_readlane(av[k], src);
      r.b = __builtin_amdgcn_readlane(bv[k], src);
    }
  }
  return r;
}

// Chunk j of the grid's order in the host plan -> (sequence, chunk of it,
// plan index).  In plan order, s is the last sequence with first[s] <= j.
// In longest-first order (a grid of several rounds), chunk j < n_full is
// the j-th full-length chunk: the last s with key[s] <= j, where key[s] =
// first[s] - (sequences before s ending in a short chunk) counts the full
// chunks before s; chunk j >= n_full is the short last chunk of sequence
// ord[j - n_full].  Every lane reads its entries of first and len and the
// mask words at once, whatever the order, so the common case takes one round
// trip to the argument memory.  Called by whole waves.
__device__ inline void host_plan_of(const HostPlan& hp, int n, int j, PlanWG& r) {
  constexpr int kR = kHostPlanSeqs / 64, kW = kHostPlanSeqs / 32;
  const int lane = threadIdx.x & 63;
  int fv[kR], lv[kR];
  // the reads do not wait for n: the tables hold kHostPlanSeqs entries
#pragma unroll
  for (int k = 0; k < kR; ++k) {
    fv[k] = hp.first[64 * k + lane];
    lv[k] = hp.len[64 * k + lane];
  }
  uint32_t mw[kW];
#pragma unroll
  for (int w = 0; w < kW; ++w) mw[w] = hp.pmask[w];
  const bool lpt = hp.lpt != 0;
  int kv[kR];
#pragma unroll
  for (int k = 0; k < kR; ++k) {
    const int i = 64 * k + lane;
    int before = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const uint32_t bits = (w < (i >> 5)) ? mw[w] : (w == (i >> 5)) ? (mw[w] & ((1u << (i & 31)) - 1u)) : 0u;
      before += __builtin_popcount(bits);
    }
    kv[k] = (i < n) ? fv[k] - (lpt ? before : 0) : 0x7FFFFFFF;
  }
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < kR; ++k) cnt += __popcll(__ballot(kv[k] <= j));
  const int s = cnt - 1, src = s & 63;
  int key = 0, len = 0, f0 = 0;
#pragma unroll
  for (int k = 0; k < kR; ++k) {
    if ((s >> 6) == k) {
      key = __builtin_amdgcn_readlane(kv[k], src);
      len = __builtin_amdgcn_readlane(lv[k], src);
      f0 = __builtin_amdgcn_readlane(fv[k], src);
    }
  }
  r.s = s;
  r.c = j - key;
  r.len = len;
  r.item = f0 + r.c;
  if (lpt && j >= hp.n_full && j < hp.first[n]) {        // a short last chunk, longest first
    const int t = hp.ord[j - hp.n_full];
    const int t0 = hp.first[t], nc = hp.first[t + 1] - t0;
    r.s = t;
    r.c = nc - 1;
    r.len = hp.len[t];
    r.item = t0 + nc - 1;
  }
  if (j < 0 || j >= hp.first[n]) r.s = -1;                 // no chunk
}

// kSrc: 0 = the host plan if p.hp.on, else the device plan; 1 = the host
// plan (a kernel instantiated for it reads the plan tables at once, without
// first waiting on the flag); 2 = the device plan.
template <int kSrc = 0>
__device__ inline PlanWG plan_of(const DecodeParams& p, int cap, int j, int s_pref, long long* sh, int* shi) {
  if (kSrc == 1 || (kSrc == 0 && p.hp.on)) {
    PlanWG r{p.hp.chunk, -1, 0, 0, -1, -1};
    host_plan_of(p.hp, p.n_seq, j, r);
    if (s_pref >= 0) r.prefix = p.hp.first[s_pref];
    return r;
  }
  PlanWG r = plan_wg(p.seq_lens, p.n_seq, cap, p.target_items, p.plan_budget, p.split_target, p.plan_slots, j,
                     s_pref, sh, shi);
  r.item = j;
  return r;
}

// seq_lens[s], from the launch arguments with a host plan.
__device__ inline int seq_len_of(const DecodeParams& p, int s) {
  return p.hp.on ? p.hp.len[s] : __builtin_amdgcn_readfirstlane(p.seq_lens[s]);
}

// Writes one merged row from the state (m, l, acc) of all its chunks.
__device__ inline void merge_write(const DecodeParams& p, int s, int h, int r, bool any_nan, float M, float lt,
                                   float4 t, int lane) {
  float4 val;
  float lse2;
  if (any_nan) {
    val = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
    lse2 = __builtin_nanf("");
  } else if (M == kNegInf) {
    val = make_float4(0.f, 0.f, 0.f, 0.f);
    lse2 = kNegInf;
  } else {
    const float inv = 1.f / lt;
    val = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
    lse2 = M + __log2f(lt);
  }
  const int tg = r / 6, g = r % 6;
  const size_t orow = static_cast<size_t>(s) * p.tok_total + tg;
  *reinterpret_cast<float4*>(p.out + (orow * kQHeads + h * kGroup + g) * kHeadDim + 4 * lane) = val;
  if (p.lse_out && lane == 0) p.lse_out[orow * kQHeads + h * kGroup + g] = lse2 * kLn2;
}

// Merges query row r of (sequence s, KV head h): nc chunks whose partial
// rows start at plan index `first`.  one_wave: this wave alone (nc <=
// kMergeBatch); else the 4 waves of the workgroup together.
__device__ inline void merge_one_row(const DecodeParams& p, int s, int h, int r, int nc, int first, bool one_wave,
                                     MergeShared& sh) {
  const int tg = r / 6, grp = tg / 8;                    // token, and its group of 8
  const int lr = r - 48 * grp;                           // row within the group's partial rows
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t item0 = static_cast<size_t>(grp) * p.part_items + static_cast<size_t>(first) * kKvHeads + h;
  const size_t prows = static_cast<size_t>(p.part_rows);
  // chunk c's row is at item0 + 4c; its address is wave-uniform (scalar
  // registers) plus this lane's 16-byte offset, and its log-sum-exp a scalar
  // load (the workspace is read-only here)
  const float* row_o = p.part_o + (item0 * prows + lr) * kHeadDim;
  typedef __attribute__((address_space(4))) const float cfloat;
  cfloat* row_l = reinterpret_cast<cfloat*>(reinterpret_cast<uintptr_t>(p.part_lse + item0 * prows + lr));
  const size_t cstride = static_cast<size_t>(kKvHeads) * prows;                 // rows between chunks
  const int c_first = one_wave ? 0 : wave, c_step = one_wave ? 1 : 4;
  // each batch: all its chunk outputs and log-sum-exps in flight at once,
  // then this wave's base m, weights 2^(x - m) and sums
  float m = kNegInf, l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  bool nan = false;
  for (int c0 = c_first; c0 < nc; c0 += c_step * kMergeBatch) {
    float4 o[kMergeBatch];
    float x[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int c = c0 + c_step * u;
      if (c < nc) {
        o[u] = reinterpret_cast<const float4*>(row_o + static_cast<size_t>(c) * cstride * kHeadDim)[lane];
        x[u] = row_l[static_cast<size_t>(c) * cstride];
      } else {
        o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        x[u] = kNegInf;
      }
    }
    float mb = m;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      nan |= (x[u] != x[u]);
      mb = fmaxf(mb, x[u]);                              // fmaxf ignores a NaN operand
    }
    if (mb == kNegInf) continue;                         // no visible key in any chunk so far
    const float a = (m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m - mb);
    acc.x *= a; acc.y *= a; acc.z *= a; acc.w *= a;
    l *= a;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float b = (x[u] == kNegInf || x[u] != x[u]) ? 0.f : __builtin_amdgcn_exp2f(x[u] - mb);
      acc.x += b * o[u].x; acc.y += b * o[u].y; acc.z += b * o[u].z; acc.w += b * o[u].w;
      l += b;
    }
    m = mb;
  }
  if (one_wave) {
    merge_write(p, s, h, r, __ballot(nan) != 0, m, l, acc, lane);
    return;
  }
  const bool any_nan = __syncthreads_or(nan);
  sh.part[wave][lane] = acc;
  if (lane == 0) {
    sh.ml[wave][0] = m;
    sh.ml[wave][1] = l;
  }
  __syncthreads();
  if (wave == 0) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sh.ml[w][0]);
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    float lt = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sh.ml[w][0];
      const float f = (mw == kNegInf) ? 0.f : exp2f(mw - M);
      const float4 u = sh.part[w][lane];
      t.x += f * u.x; t.y += f * u.y; t.z += f * u.z; t.w += f * u.w;
      lt += f * sh.ml[w][1];
    }
    merge_write(p, s, h, r, any_nan, M, lt, t, lane);
  }
}

template <bool kHost>
__device__ inline void merge_row(const DecodeParams& p, MergeShared& sh) {
  const int R = 6 * p.tok_total;                         // query rows of one (sequence, KV head)
  const int rows = kKvHeads * R;                         // query rows of a sequence
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int cap = p.bt_stride * p.page_size;
  if constexpr (kHost) {                                 // the host's plan, in the launch arguments
    const int j = blockIdx.x;
    // the last s with mfirst[s] <= j owns workgroup j (sequences without
    // merge work repeat the next one's mfirst)
    const HostHit hit = host_lookup(p.hp.mfirst, p.hp.len, p.hp.first, p.n_seq, j);
    const int s = hit.s;
    const int nc = n_chunks_of(hit.a, cap, p.hp.chunk);
    const int local = j - hit.key;
    const bool one_wave = nc <= kMergeBatch;
    const int row = one_wave ? 4 * local + wave : local;
    if (row >= rows) return;
    merge_one_row(p, s, row / R, row % R, nc, hit.b, one_wave, sh);
    return;
  }
  const int row_id = blockIdx.x;                         // one workgroup per row
  const int r = row_id % R;
  const int sh_id = row_id / R;
  const int s = sh_id / kKvHeads, h = sh_id % kKvHeads;
  int chunk, first;
  if (p.n_seq <= kHdrSeqs) {                             // the split kernel left the plan in the header
    const int32_t* hdr = reinterpret_cast<const int32_t*>(p.err);
    chunk = hdr[1];
    first = hdr[2 + s];
  } else {
    const PlanWG pl = plan_wg(p.seq_lens, p.n_seq, cap, p.target_items, p.plan_budget, p.split_target, p.plan_slots,
                              -1, s, sh.sum, sh.ints);
    chunk = pl.chunk;
    first = pl.prefix;
  }
  const int nc = n_chunks_of(seq_len_of(p, s), cap, chunk);
  if (nc <= 1) return;                                   // written by the split kernel
  const bool one_wave = nc <= kMergeBatch;
  if (one_wave && wave != 0) return;
  merge_one_row(p, s, h, r, nc, first, one_wave, sh);
}

}  // namespace dev
}  // namespace pa
