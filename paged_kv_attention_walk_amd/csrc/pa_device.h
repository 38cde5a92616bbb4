// Device helpers shared by the decode kernels: the row-address helper, the
// chunk plan, wave reductions, row decoding and the fused merge.
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

// Block-wide sum of a per-thread value (256 threads).  `sh` holds 4 slots.
__device__ inline long long block_sum(long long v, long long* sh) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  return sh[0] + sh[1] + sh[2] + sh[3];
}

// Tokens per chunk: the total live length times the KV-head count spread
// over `target` items, rounded up to the granule, at least one granule.
__device__ inline int plan_chunk(const int32_t* __restrict__ lens, int n_seq, int cap, int target,
                                 long long* sh) {
  long long acc = 0;
  for (int i = threadIdx.x; i < n_seq; i += kThreads) {
    const int L = lens[i];
    if (L > 0 && L <= cap) acc += L;
  }
  const long long total = block_sum(acc, sh);
  long long c = (total * kKvHeads + target - 1) / target;
  c = (c + kChunkGranule - 1) / kChunkGranule * kChunkGranule;
  if (c < kChunkGranule) c = kChunkGranule;
  if (c > (1ll << 30)) c = 1ll << 30;
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

// ------------------------------------------------------------ fused merge
//
// Chunks of one (sequence, KV head) are merged inside the split kernel, in a
// fixed order, by whichever workgroup arrives last:
//  level 1: chunks are grouped 16 at a time; the last of a group to finish
//           merges the group's partials (chunk order) into the slot of the
//           group's first chunk;
//  level 2: the last group to finish merges the group results (group order)
//           into the output.
// The arithmetic and its order do not depend on which workgroup runs it, so
// results are bitwise repeatable.  Arrival counters live in the workspace and
// are reset by the workgroup that consumes them.  Visibility of partials
// across workgroups (and across the per-XCD L2 caches) comes from
// device-scope fences around the counter updates: every writer fences before
// arriving, the consumer fences after it sees it is last.
//
// M = max lse; all -inf merges to 0 with lse -inf (llama.cpp pull 2,
// pd_combine fix); a NaN partial (corrupt table) gives NaN; otherwise
// out = sum_c w_c o_c / sum_c w_c with w_c = 2^(lse_c - M) (lse in base 2).
constexpr int kGroupChunks = 16;
constexpr int kMaxMergeParts = 64;

struct MergeShared {
  float w[kMaxMergeParts * 6 * kMaxQtok];
  float M[6 * kMaxQtok];
  float ws[6 * kMaxQtok];
  int flag;
};

// Merges np partials at item slots slot(k) = first_item + k * stride (k in
// order) for all R rows.  Writes the result to the output (final) or over
// slot(0).  All threads of the workgroup call it.
template <int T>
__device__ void merge_parts(const DecodeParams& p, int s, int h, size_t first_item, int stride, int np, bool final,
                            MergeShared& sh) {
  constexpr int R = 6 * T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < np * R; i += kThreads) {
    const int k = i / R, r = i % R;
    sh.w[i] = p.part_lse[(first_item + static_cast<size_t>(k) * stride) * kRowsPerItem + r];
  }
  __syncthreads();
  if (tid < R) {
    float M = kNegInf;
    bool nan = false;
    for (int k = 0; k < np; ++k) {
      const float x = sh.w[k * R + tid];
      nan |= (x != x);
      M = fmaxf(M, x);
    }
    float ws = 0.f;
    for (int k = 0; k < np; ++k) {
      const float x = sh.w[k * R + tid];
      const float wk = (M == kNegInf || x == kNegInf) ? 0.f : exp2f(x - M);
      sh.w[k * R + tid] = wk;
      ws += wk;
    }
    sh.M[tid] = nan ? __builtin_nanf("") : M;
    sh.ws[tid] = ws;
  }
  __syncthreads();
  for (int r = wave; r < R; r += 4) {
    const float M = sh.M[r], ws = sh.ws[r];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < np; ++k) {
      const float wk = sh.w[k * R + r];
      const float4 o = *reinterpret_cast<const float4*>(
          p.part_o + ((first_item + static_cast<size_t>(k) * stride) * kRowsPerItem + r) * kHeadDim + 4 * lane);
      acc.x += wk * o.x; acc.y += wk * o.y; acc.z += wk * o.z; acc.w += wk * o.w;
    }
    float4 val;
    float lse2;
    if (M != M) {
      val = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
      lse2 = __builtin_nanf("");
    } else if (M == kNegInf) {
      val = make_float4(0.f, 0.f, 0.f, 0.f);
      lse2 = kNegInf;
    } else {
      const float inv = 1.f / ws;
      val = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
      lse2 = M + __log2f(ws);
    }
    const int t = r / 6, g = r % 6;
    if (final) {
      *reinterpret_cast<float4*>(p.out + ((static_cast<size_t>(s) * T + t) * kQHeads + h * kGroup + g) * kHeadDim +
                                 4 * lane) = val;
      if (p.lse_out && lane == 0) p.lse_out[(static_cast<size_t>(s) * T + t) * kQHeads + h * kGroup + g] = lse2 * kLn2;
    } else {
      *reinterpret_cast<float4*>(p.part_o + (first_item * kRowsPerItem + r) * kHeadDim + 4 * lane) = val;
      if (lane == 0) p.part_lse[first_item * kRowsPerItem + r] = lse2;
    }
  }
}

// Arrives at counter *cnt of a group of `expected` members; returns true in
// every thread of the last arriving workgroup, which also resets the counter.
__device__ inline bool arrive_last(uint32_t* cnt, int expected, MergeShared& sh) {
  __threadfence();      // this thread's partial writes are visible device-wide before arriving
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = atomicAdd(cnt, 1u);
    const bool last = old == static_cast<uint32_t>(expected - 1);
    if (last) atomicExch(cnt, 0u);
    sh.flag = last ? 1 : 0;
  }
  __syncthreads();
  const bool last = sh.flag != 0;
  if (last) __threadfence();   // see every member's writes
  return last;
}

// After the workgroup of chunk c (of nc) of (s, h) has written its partial
// to item slot (base + c) * 4 + h: runs the two merge levels when it arrives
// last.  base = index of chunk 0 of sequence s among all (sequence, chunk) pairs.
template <int T>
__device__ void fused_merge(const DecodeParams& p, int s, int h, int c, int nc, int base, MergeShared& sh) {
  const int g = c / kGroupChunks;
  const int n_groups = (nc + kGroupChunks - 1) / kGroupChunks;
  const int g_first = g * kGroupChunks;
  const int g_size = min(kGroupChunks, nc - g_first);
  const size_t g_item = static_cast<size_t>(base + g_first) * kKvHeads + h;
  if (!arrive_last(p.cnt1 + g_item, g_size, sh)) return;
  merge_parts<T>(p, s, h, g_item, kKvHeads, g_size, n_groups == 1, sh);
  if (n_groups == 1) return;
  const size_t first_item = static_cast<size_t>(base) * kKvHeads + h;
  if (!arrive_last(p.cnt2 + first_item, n_groups, sh)) return;
  merge_parts<T>(p, s, h, first_item, kKvHeads * kGroupChunks, n_groups, true, sh);
}

}  // namespace dev
}  // namespace pa
