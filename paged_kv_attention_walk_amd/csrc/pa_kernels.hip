// HIP kernels of the paged K/V split-K decode (gfx950).
//
// Work decomposition (Luce-Org/lucebox pull 555, Summary: GQA-aware thread
// blocks, occupancy-aware context parallelism, adaptive long-context
// partitioning, stable split-softmax merge):
//  * a work item is (sequence s, KV head h, context chunk c); one workgroup
//    serves the 6 query heads x n_qtok tokens that read KV head h, so every
//    K/V row of the chunk is loaded once for all of them;
//  * chunk length is one value for the whole call, chosen from the total
//    live length and an occupancy target (a multiple of the compute-unit
//    count), so a sequence gets chunks in proportion to its length and the
//    item count stays near the target whatever the length mix;
//  * the plan is a pure function of seq_lens, n_qtok and the target, computed
//    by every workgroup from seq_lens on the device (no host round trip), and
//    identical for paged and contiguous storage;
//  * each chunk writes its normalised output and log-sum-exp; a sequence with
//    one chunk writes the final output directly, the others are combined by
//    the merge kernel (llama.cpp pull 2, pd_combine fix: a row whose keys are
//    all masked merges to 0, not 0/0).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_internal.h"

namespace pa {
namespace {

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

// Number of (sequence, chunk) pairs before sequence s.
__device__ inline int plan_prefix(const int32_t* __restrict__ lens, int s, int cap, int chunk, long long* sh) {
  long long acc = 0;
  for (int i = threadIdx.x; i < s; i += kThreads) acc += n_chunks_of(lens[i], cap, chunk);
  return static_cast<int>(block_sum(acc, sh));
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

// ------------------------------------------------------- split (VALU path)
//
// One workgroup = one (s, h, c) item; its 4 waves take 64-key groups of the
// chunk in turn.  For a group, lane j computes the logits of key j for all R
// query rows (QK), the wave updates its running max / sum (online softmax in
// base 2, the scale folded into q), and then lane l accumulates output dims
// [4l, 4l+4) over the group's keys (PV).  The 4 waves' states are combined
// through LDS at the end.
template <int KT, int VT, int T>
__global__ __launch_bounds__(kThreads) void split_valu_kernel(DecodeParams p) {
  constexpr int R = 6 * T;
  constexpr int RBK = (KT == kQ8_0) ? 272 : (KT == kQ4_0) ? 144 : 512;
  constexpr int RBV = (VT == kQ8_0) ? 272 : (VT == kQ4_0) ? 144 : 512;
  __shared__ __attribute__((aligned(16))) float q_lds[R * kHeadDim];
  __shared__ float p_lds[4][R][64];
  __shared__ const uint8_t* vrow_lds[4][64];
  __shared__ __attribute__((aligned(16))) float red[4][6][kHeadDim];
  __shared__ float ml_lds[4][R][2];
  __shared__ long long sh_sum[4];
  __shared__ int sh_loc[2];
  __shared__ int sh_bad[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cap = p.bt_stride * p.page_size;
  const int chunk = plan_chunk(p.seq_lens, p.n_seq, cap, p.target_items, sh_sum);
  const int j = blockIdx.x / kKvHeads, h = blockIdx.x % kKvHeads;
  plan_locate(p.seq_lens, p.n_seq, cap, chunk, j, sh_loc);
  const int s = sh_loc[0], c = sh_loc[1];
  if (s < 0) return;
  const int L = p.seq_lens[s];
  const int nc = n_chunks_of(L, cap, chunk);
  const size_t item = blockIdx.x;

  if (!len_ok(L, cap)) {   // corrupt length: NaN rows, nothing read
    const float nan = __builtin_nanf("");
    for (int i = tid; i < R * kHeadDim; i += kThreads) {
      const int r = i / kHeadDim, d = i % kHeadDim, t = r / 6, g = r % 6;
      p.out[((static_cast<size_t>(s) * T + t) * kQHeads + h * kGroup + g) * kHeadDim + d] = nan;
    }
    if (p.lse_out && tid < R)
      p.lse_out[(static_cast<size_t>(s) * T + tid / 6) * kQHeads + h * kGroup + tid % 6] = nan;
    if (tid == 0) atomicOr(p.err, kErrLength);
    return;
  }

  const int k0 = c * chunk;
  const int k1 = min(L, k0 + chunk);
  for (int i = tid; i < R * kHeadDim; i += kThreads) {
    const int r = i / kHeadDim, d = i % kHeadDim, t = r / 6, g = r % 6;
    q_lds[i] = p.q[((static_cast<size_t>(s) * T + t) * kQHeads + h * kGroup + g) * kHeadDim + d] * p.scale_log2;
  }
  __syncthreads();

  float m[R], l[R], o[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[r][i] = 0.f;
  }
  bool bad = false;
  const int n_groups = (k1 > k0) ? (k1 - k0 + 63) / 64 : 0;
  for (int gi = wave; gi < n_groups; gi += 4) {
    const int g0 = k0 + gi * 64;
    const int pos = g0 + lane;
    const bool in = pos < k1;
    bool ok = true;
    size_t ridx = 0;
    if (in) ridx = kv_row(p.bt, p.bt_stride, p.n_pool_blocks, p.page_size, s, h, pos, ok);
    if (__ballot(in && !ok)) bad = true;
    float sc[R];
    if (in && ok) {
      qk_row<KT, R>(p.k + ridx * RBK, q_lds, sc);
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) sc[r] = kNegInf;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int lim = L - T + r / 6;      // token t = r / 6 sees positions <= lim
      if (pos > lim) sc[r] = kNegInf;
    }
    vrow_lds[wave][lane] = p.v + ((in && ok) ? ridx * RBV : 0);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float mn = fmaxf(m[r], wave_max(sc[r]));
      const float alpha = (mn == kNegInf) ? 1.f : exp2f(m[r] - mn);
      const float pr = (sc[r] == kNegInf) ? 0.f : exp2f(sc[r] - mn);
      l[r] = l[r] * alpha + wave_sum(pr);
      m[r] = mn;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[r][i] *= alpha;
      p_lds[wave][r][lane] = pr;
    }
    wave_lds_sync();
    const int nv = min(64, k1 - g0);
    for (int jj = 0; jj < nv; ++jj) {
      float x[4];
      v_dims4<VT>(vrow_lds[wave][jj], lane, x);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float pj = p_lds[wave][r][jj];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[r][i] += pj * x[i];
      }
    }
    wave_lds_sync();
  }

  // ---- combine the 4 waves
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      ml_lds[wave][r][0] = m[r];
      ml_lds[wave][r][1] = l[r];
    }
    sh_bad[wave] = bad ? 1 : 0;
  }
  __syncthreads();
  const bool any_bad = (sh_bad[0] | sh_bad[1] | sh_bad[2] | sh_bad[3]) != 0;
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int t = 0; t < T; ++t) {
#pragma unroll
    for (int g = 0; g < 6; ++g) {
      const int r = 6 * t + g;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, ml_lds[w][r][0]);
      const float mw = ml_lds[wave][r][0];
      const float a = (mw == kNegInf) ? 0.f : exp2f(mw - M);
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][g][4 * lane + i] = o[r][i] * a;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < 6; ++g) {
      const int r = 6 * t + g;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, ml_lds[w][r][0]);
      float ltot = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = ml_lds[w][r][0];
        ltot += (mw == kNegInf) ? 0.f : ml_lds[w][r][1] * exp2f(mw - M);
      }
      const float sum = red[0][g][tid] + red[1][g][tid] + red[2][g][tid] + red[3][g][tid];
      float val = ltot > 0.f ? sum / ltot : 0.f;
      float lse2 = ltot > 0.f ? M + __log2f(ltot) : kNegInf;
      if (any_bad) {
        val = nan;
        lse2 = nan;
      }
      if (nc == 1) {
        p.out[((static_cast<size_t>(s) * T + t) * kQHeads + h * kGroup + g) * kHeadDim + tid] = val;
        if (p.lse_out && tid == 0)
          p.lse_out[(static_cast<size_t>(s) * T + t) * kQHeads + h * kGroup + g] = lse2 * kLn2;
      } else {
        p.part_o[(item * R + r) * kHeadDim + tid] = val;
        if (tid == 0) p.part_lse[item * R + r] = lse2;
      }
    }
    __syncthreads();
  }
  if (any_bad && tid == 0) atomicOr(p.err, kErrTable);
}

// ------------------------------------------------------------------ merge
//
// One workgroup per (sequence, KV head) with more than one chunk; thread d
// owns output dim d.  M = max lse_c; all -inf gives 0 (and lse -inf); a NaN
// partial (corrupt table) gives NaN; otherwise out = sum w_c o_c / sum w_c
// with w_c = 2^(lse_c - M) (lse kept in base 2 inside the kernels).
template <int T>
__global__ __launch_bounds__(kThreads) void merge_kernel(DecodeParams p) {
  constexpr int R = 6 * T;
  __shared__ long long sh_sum[4];
  const int s = blockIdx.x / kKvHeads, h = blockIdx.x % kKvHeads;
  const int cap = p.bt_stride * p.page_size;
  const int chunk = plan_chunk(p.seq_lens, p.n_seq, cap, p.target_items, sh_sum);
  const int L = p.seq_lens[s];
  const int nc = n_chunks_of(L, cap, chunk);
  if (nc <= 1) return;
  const int base = plan_prefix(p.seq_lens, s, cap, chunk, sh_sum);
  const int d = threadIdx.x;
  for (int r = 0; r < R; ++r) {
    const int t = r / 6, g = r % 6;
    float M = kNegInf;
    bool has_nan = false;
    for (int c = 0; c < nc; ++c) {
      const float x = p.part_lse[(static_cast<size_t>(base + c) * kKvHeads + h) * R + r];
      has_nan |= (x != x);
      M = fmaxf(M, x);
    }
    float val, lse2;
    if (has_nan) {
      val = lse2 = __builtin_nanf("");
    } else if (M == kNegInf) {
      val = 0.f;
      lse2 = kNegInf;
    } else {
      float ws = 0.f, acc = 0.f;
      for (int c = 0; c < nc; ++c) {
        const size_t it = static_cast<size_t>(base + c) * kKvHeads + h;
        const float w = exp2f(p.part_lse[it * R + r] - M);
        ws += w;
        acc += w * p.part_o[(it * R + r) * kHeadDim + d];
      }
      val = acc / ws;
      lse2 = M + __log2f(ws);
    }
    p.out[((static_cast<size_t>(s) * T + t) * kQHeads + h * kGroup + g) * kHeadDim + d] = val;
    if (p.lse_out && d == 0) p.lse_out[(static_cast<size_t>(s) * T + t) * kQHeads + h * kGroup + g] = lse2 * kLn2;
  }
}

// ----------------------------------------------------------- append scatter
//
// JustVugg/colibri pull 372, Summary: the appended rows arrive in one packed
// upload and a kernel scatters them into their pages.  One workgroup per row;
// 16-byte copies of each KV head's K and V row.
__global__ __launch_bounds__(kThreads) void scatter_kernel(const uint8_t* __restrict__ st, int n,
                                                           uint8_t* __restrict__ kp, uint8_t* __restrict__ vp,
                                                           int rbk, int rbv, int page_size) {
  const int i = blockIdx.x;
  const int32_t* blk = reinterpret_cast<const int32_t*>(st);
  const int b = blk[i], slot = blk[n + i];
  const uint8_t* ks = st + staging_k_off(n) + static_cast<size_t>(i) * kKvHeads * rbk;
  const uint8_t* vs = st + staging_v_off(n, rbk) + static_cast<size_t>(i) * kKvHeads * rbv;
  const int pk = rbk / 16, pv = rbv / 16;
  for (int c = threadIdx.x; c < kKvHeads * pk; c += kThreads) {
    const int hh = c / pk, off = (c % pk) * 16;
    *reinterpret_cast<uint4*>(kp + ((static_cast<size_t>(b) * kKvHeads + hh) * page_size + slot) * rbk + off) =
        *reinterpret_cast<const uint4*>(ks + hh * rbk + off);
  }
  for (int c = threadIdx.x; c < kKvHeads * pv; c += kThreads) {
    const int hh = c / pv, off = (c % pv) * 16;
    *reinterpret_cast<uint4*>(vp + ((static_cast<size_t>(b) * kKvHeads + hh) * page_size + slot) * rbv + off) =
        *reinterpret_cast<const uint4*>(vs + hh * rbv + off);
  }
}

// ------------------------------------------------------------ debug gather

__global__ __launch_bounds__(kThreads) void gather_kernel(const uint8_t* __restrict__ pool, int rb,
                                                          const int32_t* __restrict__ bt, int bt_stride,
                                                          int n_pool_blocks, int seq, int L, int page_size,
                                                          uint8_t* __restrict__ dst, int32_t* err) {
  const size_t per_row = rb / 16;
  const size_t total = static_cast<size_t>(kKvHeads) * L * per_row;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < total;
       i += static_cast<size_t>(gridDim.x) * kThreads) {
    const int piece = static_cast<int>(i % per_row);
    const size_t rowi = i / per_row;
    const int pos = static_cast<int>(rowi % L);
    const int hh = static_cast<int>(rowi / L);
    bool ok;
    const size_t ridx = kv_row(bt, bt_stride, n_pool_blocks, page_size, seq, hh, pos, ok);
    uint4 val = make_uint4(~0u, ~0u, ~0u, ~0u);
    if (ok) val = *reinterpret_cast<const uint4*>(pool + ridx * rb + piece * 16);
    *reinterpret_cast<uint4*>(dst + (static_cast<size_t>(hh) * L + pos) * rb + piece * 16) = val;
    if (!ok && err) atomicOr(err, static_cast<int32_t>(kErrTable));
  }
}

// ------------------------------------------------------------- dispatch

template <int KT, int T>
hipError_t launch_kt_t(const DecodeParams& p, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  if (e0) {
    const hipError_t e = hipEventRecord(e0, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((split_valu_kernel<KT, KT, T>), dim3(p.max_items), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (e1) {
    e = hipEventRecord(e1, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((merge_kernel<T>), dim3(p.n_seq * kKvHeads), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int KT>
hipError_t launch_kt(const DecodeParams& p, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  switch (p.n_qtok) {
    case 1: return launch_kt_t<KT, 1>(p, stream, e0, e1);
    case 2: return launch_kt_t<KT, 2>(p, stream, e0, e1);
    case 3: return launch_kt_t<KT, 3>(p, stream, e0, e1);
    case 4: return launch_kt_t<KT, 4>(p, stream, e0, e1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
  if (p.n_seq <= 0) return hipSuccess;
  if (p.k_type != p.v_type) return hipErrorInvalidValue;
  switch (p.k_type) {
    case kF16: return launch_kt<kF16>(p, stream, ev_begin, ev_end);
    case kBF16: return launch_kt<kBF16>(p, stream, ev_begin, ev_end);
    case kQ8_0: return launch_kt<kQ8_0>(p, stream, ev_begin, ev_end);
    case kQ4_0: return launch_kt<kQ4_0>(p, stream, ev_begin, ev_end);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scatter(const uint8_t* staging, int32_t n_rows, uint8_t* k_pool, uint8_t* v_pool,
                          int32_t rb_k, int32_t rb_v, int32_t page_size, hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_kernel, dim3(n_rows), dim3(kThreads), 0, stream, staging, n_rows, k_pool, v_pool,
                     rb_k, rb_v, page_size);
  return hipGetLastError();
}

hipError_t launch_gather(const uint8_t* pool, int32_t row_bytes, const int32_t* bt, int32_t bt_stride,
                         int32_t n_pool_blocks, int32_t seq, int32_t seq_len, int32_t page_size, uint8_t* dst,
                         int32_t* err_word, hipStream_t stream) {
  if (seq_len <= 0) return hipSuccess;
  const size_t total = static_cast<size_t>(kKvHeads) * seq_len * (row_bytes / 16);
  size_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(gather_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, pool, row_bytes,
                     bt, bt_stride, n_pool_blocks, seq, seq_len, page_size, dst, err_word);
  return hipGetLastError();
}

}  // namespace pa
