// Vector-ALU split kernel of the paged decode (gfx950): the fp32 reference
// path selected by PA_DECODE_VECTOR_REFERENCE.  Same work items, plan and
// merge as the matrix-core path.
//
// Built once per query-token count: compile with -DPA_T=T (1..8).  Work
// decomposition (Luce-Org/lucebox pull 555, Summary: GQA-aware thread
// blocks, occupancy-aware context parallelism): one workgroup per (sequence,
// KV head, context chunk) serves the 6 query heads x T tokens reading that
// KV head.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstdint>

#include "pa_device.h"
#include "pa_internal.h"

#ifndef PA_T
#error "build with -DPA_T=<query tokens>"
#endif

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
  __shared__ long long sh_sum[kPlanShared];
  __shared__ int sh_loc[4];
  __shared__ int sh_bad[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cap = p.bt_stride * p.page_size;

  const int grp = blockIdx.x % p.n_groups;           // token group fastest
  const int item_id = blockIdx.x / p.n_groups;
  const int tok0 = p.tok0 + T * grp;                   // first token of this workgroup's rows
  const int j = item_id / kKvHeads, h = item_id % kKvHeads;
  const PlanWG pl = plan_of(p, cap, j, -1, sh_sum, sh_loc);
  const int chunk = pl.chunk, s = pl.s, c = pl.c;
  if (s < 0) return;
  if (tid == 0 && c == 0 && h == 0 && tok0 == 0) {      // the plan, for the merge kernel
    int32_t* hdr = reinterpret_cast<int32_t*>(p.err);
    if (s < kHdrSeqs) hdr[2 + s] = j;
    if (s == 0) hdr[1] = chunk;
  }
  const int L = p.hp.on ? pl.len : seq_len_of(p, s);
  const int nc = n_chunks_of(L, cap, chunk);
  const size_t part =
      (static_cast<size_t>(tok0 / 8) * p.part_items + static_cast<size_t>(pl.item) * kKvHeads + h) * p.part_rows +
      6 * (tok0 % 8);
  const size_t orow = static_cast<size_t>(s) * p.tok_total + tok0;   // output row of the group's token 0

  if (!len_ok(L, cap)) {   // corrupt length: NaN rows, nothing read
    const float nan = __builtin_nanf("");
    for (int i = tid; i < R * kHeadDim; i += kThreads) {
      const int r = i / kHeadDim, d = i % kHeadDim, t = r / 6, g = r % 6;
      p.out[((orow + t) * kQHeads + h * kGroup + g) * kHeadDim + d] = nan;
    }
    if (p.lse_out && tid < R) p.lse_out[(orow + tid / 6) * kQHeads + h * kGroup + tid % 6] = nan;
    if (tid == 0) atomicOr(p.err, kErrLength);
    return;
  }

  // token t of the group sits at position lim_base + t and sees the
  // positions up to it; keys past the group's last token are skipped
  const int lim_base = L - p.tok_total + tok0;
  const int k0 = c * chunk;
  const int k1 = max(k0, min(min(L, k0 + chunk), lim_base + T));
  for (int i = tid; i < R * kHeadDim; i += kThreads) {
    const int r = i / kHeadDim, d = i % kHeadDim, t = r / 6, g = r % 6;
    q_lds[i] = p.q[((orow + t) * kQHeads + h * kGroup + g) * kHeadDim + d] * p.scale_log2;
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
      const int lim = lim_base + r / 6;   // token t = r / 6 sees positions <= lim
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
        p.out[((orow + t) * kQHeads + h * kGroup + g) * kHeadDim + tid] = val;
        if (p.lse_out && tid == 0) p.lse_out[(orow + t) * kQHeads + h * kGroup + g] = lse2 * kLn2;
      } else {
        p.part_o[(part + r) * kHeadDim + tid] = val;
        if (tid == 0) p.part_lse[part + r] = lse2;
      }
    }
    __syncthreads();
  }
  if (any_bad && tid == 0) atomicOr(p.err, kErrTable);
}

template <int KT, int VT>
hipError_t launch_kvt(const DecodeParams& p, const SplitLaunch& l) {
  const dim3 grid(static_cast<unsigned>(grid_items(p)) * static_cast<unsigned>(p.n_groups));
  void* args[] = {const_cast<DecodeParams*>(&p)};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(&split_valu_kernel<KT, VT, PA_T>), grid, dim3(kThreads), args, 0,
                            l.stream, l.start, l.stop, 0);
}

template <int KT>
hipError_t launch_kt(const DecodeParams& p, const SplitLaunch& l) {
  switch (p.v_type) {
    case kF16: return launch_kvt<KT, kF16>(p, l);
    case kBF16: return launch_kvt<KT, kBF16>(p, l);
    case kQ8_0: return launch_kvt<KT, kQ8_0>(p, l);
    case kQ4_0: return launch_kvt<KT, kQ4_0>(p, l);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

template <>
hipError_t launch_split_valu_t<PA_T>(const DecodeParams& p, const SplitLaunch& l) {
  switch (p.k_type) {
    case kF16: return launch_kt<kF16>(p, l);
    case kBF16: return launch_kt<kBF16>(p, l);
    case kQ8_0: return launch_kt<kQ8_0>(p, l);
    case kQ4_0: return launch_kt<kQ4_0>(p, l);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
