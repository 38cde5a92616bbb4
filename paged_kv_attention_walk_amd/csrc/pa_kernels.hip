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
//  * the plan is a pure function of seq_lens, n_qtok and the target, and
//    identical for paged and contiguous storage.  Every workgroup computes it
//    from seq_lens on the device (no host round trip), or, when the caller
//    also passes the lengths on the host, the host computes it with the same
//    arithmetic and it arrives with the launch arguments;
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

// ------------------------------------------------------- read ceiling
//
// Reads n16 16-byte words once each and folds them with xor; one word per
// wave goes to `sink` so that nothing is optimised away.  The HBM read rate
// the decode kernels are compared against.  U loads are in flight per lane.
// Access: grid-stride (consecutive lanes, then waves, then workgroups read
// adjacent words; a step of the loop covers the whole grid), or per-slice
// (each workgroup streams one contiguous share of the buffer in 4 KB
// steps, as a split-K work item streams its chunk).  Loads land in registers,
// or with kLds go straight to LDS (global_load_lds_dwordx4): the data is not
// used there, every load of a wave overwrites the wave's one 1 KB slot.
template <int U, bool kLds, bool kSlice>
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint4* __restrict__ src, size_t n16,
                                                              uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) uint32_t slot[kLds ? kThreads * 4 : 4];
  size_t i, end, stride;
  if constexpr (kSlice) {
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t first = static_cast<size_t>(blockIdx.x) * per;
    end = first + per < n16 ? first + per : n16;
    i = first + threadIdx.x;
    stride = kThreads;
  } else {
    end = n16;
    i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
    stride = static_cast<size_t>(gridDim.x) * kThreads;
  }
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < end; i += U * stride) {
    if constexpr (kLds) {
      typedef __attribute__((address_space(3))) void lds_void;
      lds_void* dst = reinterpret_cast<lds_void*>(reinterpret_cast<uintptr_t>(slot) + (threadIdx.x >> 6) * 1024);
#pragma unroll
      for (int u = 0; u < U; ++u) __builtin_amdgcn_global_load_lds(src + i + u * stride, dst, 16, 0, 0);
    } else {
      uint4 a[U];
#pragma unroll
      for (int u = 0; u < U; ++u) a[u] = src[i + u * stride];
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
    }
  }
  for (; i < end; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if constexpr (kLds) {
    __builtin_amdgcn_s_waitcnt(0);      // every direct-to-LDS load has landed
    __syncthreads();
    acc ^= slot[threadIdx.x];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = acc;
}

// ------------------------------------------------------------- dispatch

// One instantiation per plan source, so that a host-planned merge reads its
// plan tables without first waiting on the flag that selects them.
template <bool kHost>
__global__ __launch_bounds__(kThreads) void merge_kernel(DecodeParams p) {
  __shared__ MergeShared sh;
  merge_row<kHost>(p, sh);
}

hipError_t launch_merge(const DecodeParams& p, hipStream_t stream) {
  // the host's plan: the compact grid; else one workgroup per query row
  const unsigned wgs = p.hp.on ? static_cast<unsigned>(p.hp.mfirst[p.n_seq])
                               : static_cast<unsigned>(p.n_seq) * kKvHeads * 6 * static_cast<unsigned>(p.tok_total);
  if (wgs == 0) return hipSuccess;
  const dim3 grid(wgs), block(kThreads);
  if (p.hp.on)
    hipLaunchKernelGGL(merge_kernel<true>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(merge_kernel<false>, grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_split(const DecodeParams& p, const SplitLaunch& l) {
  const bool valu = p.engine == 1;
  switch (p.n_qtok) {
    case 1: return valu ? launch_split_valu_t<1>(p, l) : launch_split_mfma_t<1>(p, l);
    case 2: return valu ? launch_split_valu_t<2>(p, l) : launch_split_mfma_t<2>(p, l);
    case 3: return valu ? launch_split_valu_t<3>(p, l) : launch_split_mfma_t<3>(p, l);
    case 4: return valu ? launch_split_valu_t<4>(p, l) : launch_split_mfma_t<4>(p, l);
    case 5: return valu ? launch_split_valu_t<5>(p, l) : launch_split_mfma_t<5>(p, l);
    // the matrix-core path runs at most five tokens per launch group
    case 6: return valu ? launch_split_valu_t<6>(p, l) : hipErrorInvalidValue;
    case 7: return valu ? launch_split_valu_t<7>(p, l) : hipErrorInvalidValue;
    case 8: return valu ? launch_split_valu_t<8>(p, l) : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int split_wgs_per_cu(int k_type, int v_type, int n_qtok, int engine) {
  if (engine == 1) return n_qtok <= 4 ? 2 : 1;   // vector reference path (per-lane rows grow with n_qtok)
  switch (n_qtok) {
    case 1: return split_mfma_wgs_t<1>(k_type, v_type);
    case 2: return split_mfma_wgs_t<2>(k_type, v_type);
    case 3: return split_mfma_wgs_t<3>(k_type, v_type);
    case 4: return split_mfma_wgs_t<4>(k_type, v_type);
    case 5: return split_mfma_wgs_t<5>(k_type, v_type);
    case 6: return split_mfma_wgs_t<3>(k_type, v_type);   // two groups of three
    default: return split_mfma_wgs_t<4>(k_type, v_type);  // seven and eight: groups of four
  }
}

// ev_begin / ev_end (optional) are attached to the split launches: begin to
// the first, end to the last (the vector path takes two when the token
// count is not a multiple of its group size), so they time the split
// kernels' execution.
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
  if (p.n_seq <= 0) return hipSuccess;
  const int gt = p.group_tok;
  if (gt < 1 || gt > kMaxQtok) return hipErrorInvalidValue;
  // the matrix-core kernels mask the missing tokens of a partial last group:
  // every group in one launch; the vector path runs the full groups in one
  // launch and the rest in another
  const bool whole = p.engine == 0;
  const int full = whole ? (p.tok_total + gt - 1) / gt : p.tok_total / gt;
  const int rest = whole ? 0 : p.tok_total % gt;
  hipError_t e = hipSuccess;
  if (full > 0) {
    DecodeParams a = p;
    a.n_qtok = gt;
    a.n_groups = full;
    a.tok0 = 0;
    e = launch_split(a, SplitLaunch{stream, ev_begin, rest > 0 ? nullptr : ev_end});
  }
  if (e == hipSuccess && rest > 0) {
    DecodeParams b = p;
    b.n_qtok = rest;
    b.n_groups = 1;
    b.tok0 = full * gt;
    e = launch_split(b, SplitLaunch{stream, full > 0 ? nullptr : ev_begin, ev_end});
  }
  if (e != hipSuccess) return e;
  if (p.hp.on && !p.hp.any_multi) return hipSuccess;   // every sequence wrote its rows directly
  return launch_merge(p, stream);
}

hipError_t launch_scatter(const uint8_t* staging, int32_t n_rows, uint8_t* k_pool, uint8_t* v_pool,
                          int32_t rb_k, int32_t rb_v, int32_t page_size, hipStream_t stream) {
  if (n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_kernel, dim3(n_rows), dim3(kThreads), 0, stream, staging, n_rows, k_pool, v_pool,
                     rb_k, rb_v, page_size);
  return hipGetLastError();
}

template <bool kLds, bool kSlice>
hipError_t launch_read_probe_u(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, int32_t unroll,
                               hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(blocks)), block(kThreads);
  const uint4* s = static_cast<const uint4*>(src);
  switch (unroll) {
    case 1: hipLaunchKernelGGL((read_probe_kernel<1, kLds, kSlice>), grid, block, 0, stream, s, bytes / 16, sink); break;
    case 2: hipLaunchKernelGGL((read_probe_kernel<2, kLds, kSlice>), grid, block, 0, stream, s, bytes / 16, sink); break;
    case 4: hipLaunchKernelGGL((read_probe_kernel<4, kLds, kSlice>), grid, block, 0, stream, s, bytes / 16, sink); break;
    case 8: hipLaunchKernelGGL((read_probe_kernel<8, kLds, kSlice>), grid, block, 0, stream, s, bytes / 16, sink); break;
    case 16: hipLaunchKernelGGL((read_probe_kernel<16, kLds, kSlice>), grid, block, 0, stream, s, bytes / 16, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, int32_t unroll,
                             bool to_lds, bool slice, hipStream_t stream) {
  if (to_lds) return slice ? launch_read_probe_u<true, true>(src, bytes, sink, blocks, unroll, stream)
                           : launch_read_probe_u<true, false>(src, bytes, sink, blocks, unroll, stream);
  return slice ? launch_read_probe_u<false, true>(src, bytes, sink, blocks, unroll, stream)
               : launch_read_probe_u<false, false>(src, bytes, sink, blocks, unroll, stream);
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
