// Device-side append with fused encoding (gfx950).
//
// JustVugg/colibri pull 372, "cuda: keep paged ragged KV resident across
// decode steps", Summary: only the newly appended K/V rows move, and a
// scatter kernel puts each into its page.  Here the rows are already in
// device memory as float32 (or bf16 / f16) values, as a K/V projection
// leaves them, and the kernel encodes them into the pool's K and V encodings
// on the way: no host staging and no separate quantise pass over HBM.
//
// Encodings (the workload definitions of Q4_0 and Q8_0: fp16 scale
// d = max|x|/8 resp. max|x|/127 over a block of 32 values):
//  * d = fp16(max|x| / q), the division in float32, rounded to nearest even;
//  * codes against the stored scale: c = round(x * r), r = 1 / float(d) in
//    float32, the product a float32 multiply, halves away from zero
//    (roundf); Q8_0 clips to [-127, 127], Q4_0 stores c + 8 clipped to
//    [0, 15]; a zero block stores d = 0 and codes 8 / 0;
//  * F16 / BF16: nearest value, ties to even.
//
// One workgroup per (row, K or V); its wave w encodes KV head w.  Lane l
// holds values [4l, 4l + 4) of the head's 256, so a block of 32 is 8
// adjacent lanes: the block max is three xor shuffles.  Block formats are
// assembled in LDS (their 18- and 34-byte blocks put codes at 2-byte
// aligned offsets) and leave with 16-byte stores; the 2-byte formats are
// stored straight from registers.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreadsAppend = 256;
constexpr uint32_t kErrAppend = 4u;   // PA_DEVERR_APPEND

template <int ST>
__device__ __forceinline__ float4 load4(const void* src, size_t elem) {
  if constexpr (ST == kSrcF32) {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(src) + elem);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + elem);
    const uint32_t h[4] = {w.x & 0xffffu, w.x >> 16, w.y & 0xffffu, w.y >> 16};
    float f[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if constexpr (ST == kSrcBF16) {
        f[m] = __uint_as_float(h[m] << 16);
      } else {
        f[m] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h[m])));
      }
    }
    return make_float4(f[0], f[1], f[2], f[3]);
  }
}

__device__ __forceinline__ uint32_t to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

__device__ __forceinline__ uint32_t to_bf16_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  if ((b & 0x7fffffffu) > 0x7f800000u) return (b >> 16) | 0x40u;   // NaN stays a (quiet) NaN
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float block_max8(float v) {
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  return v;
}

// Stored fp16 scale of a block (bits) and the float32 reciprocal used for
// its codes.
__device__ __forceinline__ void block_scale(float amax, float q, uint32_t& d_bits, float& r) {
  const _Float16 d = static_cast<_Float16>(amax / q);
  d_bits = __builtin_bit_cast(uint16_t, d);
  const float df = static_cast<float>(d);
  r = (df != 0.0f) ? 1.0f / df : 0.0f;
}

__device__ __forceinline__ void lds_u16(uint8_t* p, uint32_t v) {
  *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(v);
}

struct AppendArgs {
  const void* src[2];        // K, V source rows [n][4][256]
  uint8_t* pool[2];          // K, V pools
  int32_t type[2];           // their encodings
  int32_t rb[2];             // their row bytes
  const int32_t* dst_block;  // [n]
  const int32_t* dst_slot;   // [n]
  uint32_t* err;
  int32_t n_rows, n_blocks, page_size;
};

template <int ST>
__global__ __launch_bounds__(kThreadsAppend) void append_encode_kernel(AppendArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t rows[kKvHeads][512];
  const int i = blockIdx.x, kv = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = a.dst_block[i], s = a.dst_slot[i];
  if (b < 0 || b >= a.n_blocks || s < 0 || s >= a.page_size) {      // uniform over the workgroup
    if (threadIdx.x == 0 && kv == 0) atomicOr(a.err, kErrAppend);
    return;
  }
  const int t = a.type[kv], rb = a.rb[kv];
  uint8_t* dst = a.pool[kv] + ((static_cast<size_t>(b) * kKvHeads + wave) * a.page_size + s) * rb;
  const float4 x = load4<ST>(a.src[kv], (static_cast<size_t>(i) * kKvHeads + wave) * kHeadDim + 4 * lane);
  const float xv[4] = {x.x, x.y, x.z, x.w};

  if (t == kF16 || t == kBF16) {
    uint32_t h[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) h[m] = (t == kF16) ? to_f16_bits(xv[m]) : to_bf16_bits(xv[m]);
    *reinterpret_cast<uint2*>(dst + 8 * lane) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    return;
  }

  const int q = lane >> 3, k = lane & 7;   // block q of the row, lane k of the block
  const float amax = block_max8(fmaxf(fmaxf(fabsf(xv[0]), fabsf(xv[1])), fmaxf(fabsf(xv[2]), fabsf(xv[3]))));
  uint8_t* row = rows[wave];
  uint32_t d_bits;
  float r;
  if (t == kQ8_0) {
    block_scale(amax, 127.0f, d_bits, r);
    uint32_t c[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float v = fminf(fmaxf(roundf(xv[m] * r), -127.0f), 127.0f);
      c[m] = static_cast<uint32_t>(static_cast<int32_t>(v)) & 0xffu;
    }
    uint8_t* blk = row + 34 * q;
    if (k == 0) lds_u16(blk, d_bits);
    lds_u16(blk + 2 + 4 * k, c[0] | (c[1] << 8));
    lds_u16(blk + 4 + 4 * k, c[2] | (c[3] << 8));
  } else {   // kQ4_0
    block_scale(amax, 8.0f, d_bits, r);
    uint32_t nib = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float v = fminf(fmaxf(roundf(xv[m] * r) + 8.0f, 0.0f), 15.0f);
      nib |= static_cast<uint32_t>(v) << (4 * m);
    }
    // lanes k < 4 hold elements 4k.. of the block, lanes k + 4 the elements
    // 16 higher: byte j takes element j low and element j + 16 high
    const uint32_t hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(nib), 4));
    uint8_t* blk = row + 18 * q;
    if (k == 0) lds_u16(blk, d_bits);
    if (k < 4) {
      uint32_t by[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) by[m] = ((nib >> (4 * m)) & 15u) | (((hi >> (4 * m)) & 15u) << 4);
      lds_u16(blk + 2 + 4 * k, by[0] | (by[1] << 8));
      lds_u16(blk + 4 + 4 * k, by[2] | (by[3] << 8));
    }
  }
  __syncthreads();
  if (lane < rb / 16) *reinterpret_cast<uint4*>(dst + 16 * lane) = *reinterpret_cast<const uint4*>(row + 16 * lane);
}

}  // namespace

hipError_t launch_append_encode(const AppendLaunch& l, hipStream_t stream) {
  if (l.n_rows <= 0) return hipSuccess;
  AppendArgs a;
  a.src[0] = l.k_src;
  a.src[1] = l.v_src;
  a.pool[0] = l.k_pool;
  a.pool[1] = l.v_pool;
  a.type[0] = l.k_type;
  a.type[1] = l.v_type;
  a.rb[0] = row_bytes_of(l.k_type);
  a.rb[1] = row_bytes_of(l.v_type);
  a.dst_block = l.dst_block;
  a.dst_slot = l.dst_slot;
  a.err = l.err;
  a.n_rows = l.n_rows;
  a.n_blocks = l.n_blocks;
  a.page_size = l.page_size;
  const dim3 grid(static_cast<unsigned>(l.n_rows), 2);
  switch (l.src_type) {
    case kSrcF32: hipLaunchKernelGGL(append_encode_kernel<kSrcF32>, grid, dim3(kThreadsAppend), 0, stream, a); break;
    case kSrcBF16: hipLaunchKernelGGL(append_encode_kernel<kSrcBF16>, grid, dim3(kThreadsAppend), 0, stream, a); break;
    case kSrcF16: hipLaunchKernelGGL(append_encode_kernel<kSrcF16>, grid, dim3(kThreadsAppend), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
