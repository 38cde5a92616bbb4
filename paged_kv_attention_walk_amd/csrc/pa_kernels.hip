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
//    the merge kernel.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

using namespace dev;

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

  // ---- combine the 4 waves, write this chunk's rows, then merge
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
        p.part_o[(item * kRowsPerItem + r) * kHeadDim + tid] = val;
        if (tid == 0) p.part_lse[item * kRowsPerItem + r] = lse2;
      }
    }
    __syncthreads();
  }
  if (any_bad && tid == 0) atomicOr(p.err, kErrTable);
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

template <int T>
__global__ __launch_bounds__(kThreads) void merge_kernel(DecodeParams p) {
  __shared__ MergeShared sh;
  merge_row<T>(p, sh);
}

hipError_t launch_merge(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid(p.n_seq * kKvHeads * 6 * p.n_qtok), block(kThreads);
  switch (p.n_qtok) {
    case 1: hipLaunchKernelGGL((merge_kernel<1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((merge_kernel<2>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((merge_kernel<3>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((merge_kernel<4>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KT, int VT>
hipError_t launch_valu_kvt(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid(p.max_items), block(kThreads);
  switch (p.n_qtok) {
    case 1: hipLaunchKernelGGL((split_valu_kernel<KT, VT, 1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((split_valu_kernel<KT, VT, 2>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((split_valu_kernel<KT, VT, 3>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((split_valu_kernel<KT, VT, 4>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KT>
hipError_t launch_valu_kt(const DecodeParams& p, hipStream_t stream) {
  switch (p.v_type) {
    case kF16: return launch_valu_kvt<KT, kF16>(p, stream);
    case kBF16: return launch_valu_kvt<KT, kBF16>(p, stream);
    case kQ8_0: return launch_valu_kvt<KT, kQ8_0>(p, stream);
    case kQ4_0: return launch_valu_kvt<KT, kQ4_0>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_split_valu(const DecodeParams& p, hipStream_t stream) {
  switch (p.k_type) {
    case kF16: return launch_valu_kt<kF16>(p, stream);
    case kBF16: return launch_valu_kt<kBF16>(p, stream);
    case kQ8_0: return launch_valu_kt<kQ8_0>(p, stream);
    case kQ4_0: return launch_valu_kt<kQ4_0>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int split_wgs_per_cu(int k_type, int v_type, int n_qtok, int engine) {
  if (engine == 1) return 2;     // vector reference path: 256 threads, modest registers
  return split_mfma_wgs_per_cu(k_type, v_type, n_qtok);
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
  if (p.n_seq <= 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if (ev_begin) e = hipEventRecord(ev_begin, stream);
  if (e != hipSuccess) return e;
  e = (p.engine == 1) ? launch_split_valu(p, stream) : launch_split_mfma(p, stream);
  if (e != hipSuccess) return e;
  if (ev_end) e = hipEventRecord(ev_end, stream);
  if (e != hipSuccess) return e;
  return launch_merge(p, stream);
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
