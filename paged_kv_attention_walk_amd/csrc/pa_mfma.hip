// Matrix-core split kernel of the paged decode (gfx950).
//
// Same work items, plan and merge kernel as the vector path; the per-chunk
// math runs on v_mfma_f32_16x16x32_{f16,bf16}.  One workgroup = one
// (sequence, KV head, chunk); its 4 waves take 32-key tiles of the chunk in
// turn, each wave with its own running max / sum / output.
//
// Per 32-key tile (two 16-key halves, each inside one page, so the block
// table is read once per half -- llama.cpp pull 2, page-table commit, resolves
// its table once per chunk of keys rather than per key):
//  * QK^T as S^T = K Q^T: the A operand is 16 keys x 32 dims of one
//    quantisation block, loaded from HBM straight into operand registers (a
//    lane holds 8 dims of one key; Q4_0 rows instead arrive as contiguous
//    16-byte pieces, are kept raw in LDS and read from there) and converted
//    in-register to exact f16 values (codes for Q8_0 / Q4_0); the B operand
//    is the 6*T query rows of the
//    KV head (in 16-column tiles), split as q = q_hi + q_lo in f16 (bf16 for
//    BF16 K) so the products carry ~22 bits.  For Q8_0 / Q4_0 the block scale
//    is applied per key to the fp32 result of each block's MFMA, so codes
//    stay exact (llama.cpp pull 2, LDS-read commit, converts quants in
//    registers; here the fp16 scale never touches an f16 operand).
//  * online softmax in base 2 (log2 e folded into q), rows spread over the
//    4 lanes that hold them;
//  * PV as O^T = V^T P^T: V rows are staged in the wave's LDS (codes and
//    scales split apart), and the gfx950 LDS transpose reads
//    (ds_read_b64_tr_b4 / _b8 / _b16) deliver the V^T operand -- 8 keys of one
//    dim per lane -- in one read per block (Q4_0), per 16 dims (Q8_0) or two
//    per 16 dims (F16 / BF16).  For Q8_0 / Q4_0 the operand is the code
//    times the per-key block scale, split exactly into f16 hi + lo parts (a
//    code times an fp16 scale has at most 19 significant bits), and the
//    probabilities are split hi + lo like q.
// Accumulation is fp32 throughout.
//
// This source is built once per query-token count T (-DPA_T=T, 1..5; a call
// of more tokens runs as token groups of at most four): the 6T query rows of
// a KV head take ceil(6T/16) B tiles of 16 columns, and a last tile of at
// most 8 rows packs the hi and lo parts into one tile (one, three and four
// tokens).
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cstdint>

#include "pa_device.h"
#include "pa_internal.h"

#ifndef PA_T
#error "build with -DPA_T=<query tokens>"
#endif
static_assert(PA_T >= 1 && PA_T <= 5, "matrix-core launch groups hold 1..5 tokens");

namespace pa {
namespace {

using namespace dev;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef int32_t i2 __attribute__((ext_vector_type(2)));
typedef short s4 __attribute__((ext_vector_type(4)));
// dword-aligned multi-dword loads from rows whose start is 4-byte aligned
typedef uint32_t u4a __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u2a __attribute__((ext_vector_type(2), aligned(4)));

typedef __attribute__((address_space(3))) i2 lds_i2;
typedef __attribute__((address_space(3))) s4 lds_s4;

template <int KT>
struct Fmt {
  static constexpr bool kQuant = (KT == kQ8_0 || KT == kQ4_0);
  static constexpr bool kBf = (KT == kBF16);
  static constexpr int kRow = (KT == kQ8_0) ? 272 : (KT == kQ4_0) ? 144 : 512;   // bytes per row
  static constexpr int kBlk = (KT == kQ8_0) ? 34 : 18;                           // bytes per quant block
  static constexpr int kCodes = (KT == kQ8_0) ? 32 : 16;                         // code bytes per block
  // LDS stride of one staged V key: codes (quant) or the row, plus 16 bytes
  // so that keys 4 apart fall in different banks.
  static constexpr int kVks = kQuant ? 8 * kCodes + 16 : 512 + 16;
  static constexpr int kVtile = 32 * kVks;                                     // 32 keys
  // Q4_0 K rows are fetched as contiguous 16-byte pieces and kept raw in LDS
  // (the operands are read there); other types load K in operand layout.
  static constexpr bool kKStage = (KT == kQ4_0);
  static constexpr int kKraw = kKStage ? 32 * kRow : 0;
  // A V buffer: V codes, then (quant) V scales as f16 (512 B).  The K area
  // (quant): the key bias (f32 [2][16]: 0 for a visible key, -inf past the
  // chunk end or for a dead half), K scales (f32 [2][8][16]), raw K rows.
  static constexpr int kVbuf = kVtile + (kQuant ? 512 : 0);
  static constexpr int kKBias = 0;
  static constexpr int kKScale = 512;
  static constexpr int kKRaw = 1536;
  static constexpr int kKarea = kQuant ? kKRaw + kKraw : 0;
};

__device__ inline f4 mma(u4 a, u4 b, f4 c, bool bf) {
  if (bf)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
}

// f16 pair (a, b) -> packed bits
__device__ inline uint32_t pack_h(_Float16 a, _Float16 b) {
  return static_cast<uint32_t>(__builtin_bit_cast(unsigned short, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(unsigned short, b)) << 16);
}
__device__ inline uint32_t pack_bf(__bf16 a, __bf16 b) {
  return static_cast<uint32_t>(__builtin_bit_cast(unsigned short, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(unsigned short, b)) << 16);
}

// Splits 8 floats into hi + lo 16-bit operands (f16, or bf16 when bf).
__device__ inline void split8(const float (&x)[8], u4& hi, u4& lo, bool bf) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = x[2 * k], b = x[2 * k + 1];
    if (bf) {
      const __bf16 ha = static_cast<__bf16>(a), hb = static_cast<__bf16>(b);
      hi[k] = pack_bf(ha, hb);
      lo[k] = pack_bf(static_cast<__bf16>(a - static_cast<float>(ha)), static_cast<__bf16>(b - static_cast<float>(hb)));
    } else {
      const _Float16 ha = static_cast<_Float16>(a), hb = static_cast<_Float16>(b);
      hi[k] = pack_h(ha, hb);
      lo[k] = pack_h(static_cast<_Float16>(a - static_cast<float>(ha)), static_cast<_Float16>(b - static_cast<float>(hb)));
    }
  }
}

__device__ inline uint32_t pkrtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// 8 floats as f16 hi + lo parts with round-toward-zero conversions: hi =
// rtz(x) and lo = rtz(x - hi), where x - hi is exact in f32 (hi keeps the
// leading 11 bits of x), so hi + lo holds x to about 22 bits.  With `m` = 0
// a lane gets hi in `lo` as well, with m = -1 the remainder: the one-token
// packing takes its part with no select (lanes n < 8 hi, n >= 8 lo).
__device__ inline void split8_rtz(const float (&x)[8], u4& hi, u4& lo, float m) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t h = pkrtz(x[2 * k], x[2 * k + 1]);
    hi[k] = h;
    const h2 hv = __builtin_bit_cast(h2, h);
    lo[k] = pkrtz(__builtin_fmaf(static_cast<float>(hv[0]), m, x[2 * k]),
                  __builtin_fmaf(static_cast<float>(hv[1]), m, x[2 * k + 1]));
  }
}

// (x & mask) | (0x64006400 & ~mask): one bit-field insert.
__device__ inline uint32_t bfi(uint32_t mask, uint32_t x, uint32_t y) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(x), "v"(y));
  return r;
}

// (x & mask) | 0x64006400 read as two f16 (1024 + field), minus `sub` each.
__device__ inline uint32_t nib2h(uint32_t x, uint32_t mask, float sub) {
  const uint32_t u = bfi(mask, x, 0x64006400u);
  h2 v = __builtin_bit_cast(h2, u);
  const h2 s = {static_cast<_Float16>(sub), static_cast<_Float16>(sub)};
  v = v - s;
  return __builtin_bit_cast(uint32_t, v);
}

// (x & 0x00F000F0) | 0x64006400 read as two f16 (1024 + 16 field), times
// 1/16 minus 72: the field minus 8, exactly (one fused multiply-add).
__device__ inline uint32_t nib2h_hi(uint32_t x) {
  const uint32_t u = bfi(0x00F000F0u, x, 0x64006400u);
  const h2 v = __builtin_bit_cast(h2, u);
  const h2 k = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
  const h2 c = {static_cast<_Float16>(-72.f), static_cast<_Float16>(-72.f)};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(v, k, c));
}

// 8 nibbles (bits 4k, k = 0..7) -> f16 operand c - 8, element order
// k = 0,4,1,5,2,6,3,7.  With X16, elements of odd k hold 16 (c - 8) instead
// (the partner operand then carries 1/16); without, they are brought down
// by a fused multiply-add.  No shift for odd k either way.
template <bool X16>
__device__ inline u4 q4_operand(uint32_t x) {
  const uint32_t y = x >> 8;
  u4 a;
  a[0] = nib2h(x, 0x000F000Fu, 1032.f);                       // k = 0, 4
  a[2] = nib2h(y, 0x000F000Fu, 1032.f);                       // k = 2, 6
  if constexpr (X16) {
    a[1] = nib2h(x, 0x00F000F0u, 1152.f);                     // k = 1, 5: 16 (c - 8)
    a[3] = nib2h(y, 0x00F000F0u, 1152.f);                     // k = 3, 7
  } else {
    a[1] = nib2h_hi(x);                                       // k = 1, 5
    a[3] = nib2h_hi(y);                                       // k = 3, 7
  }
  return a;
}

// 8 signed bytes (two dwords) -> f16 operand, element order 0,2,1,3,4,6,5,7.
__device__ inline u4 q8_operand(uint32_t x0, uint32_t x1) {
  const uint32_t y0 = x0 ^ 0x80808080u, y1 = x1 ^ 0x80808080u;
  u4 a;
  a[0] = nib2h(y0, 0x00FF00FFu, 1152.f);
  a[1] = nib2h(y0 >> 8, 0x00FF00FFu, 1152.f);
  a[2] = nib2h(y1, 0x00FF00FFu, 1152.f);
  a[3] = nib2h(y1 >> 8, 0x00FF00FFu, 1152.f);
  return a;
}

__device__ inline uint32_t funnel16(uint32_t lo, uint32_t hi) { return (lo >> 16) | (hi << 16); }

// Cross-lane butterflies without LDS.  The value of lane l ^ 8 (inside each
// 16-lane row: a rotation by 8), and x op x' for the partner l ^ 16 or
// l ^ 32 from the gfx950 row / half swaps: the two swapped copies hold own
// and partner values in some order, and op is commutative, so every lane of
// a pair gets the same result.
__device__ inline float lane_xor8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}
__device__ inline float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_bit_cast(float, static_cast<unsigned>(r[0])) + __builtin_bit_cast(float, static_cast<unsigned>(r[1]));
}
__device__ inline float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_bit_cast(float, static_cast<unsigned>(r[0])) + __builtin_bit_cast(float, static_cast<unsigned>(r[1]));
}
__device__ inline float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, static_cast<unsigned>(r[0])), __builtin_bit_cast(float, static_cast<unsigned>(r[1])));
}
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, static_cast<unsigned>(r[0])), __builtin_bit_cast(float, static_cast<unsigned>(r[1])));
}

// a * d as hi + lo f16 pairs, exactly: a holds small integers (codes) and d
// fp16 scales, so the product has at most 19 significant bits; hi is its f16
// rounding and lo = fma(a, d, -hi) the remainder, which f16 holds exactly.
__device__ inline uint32_t mul_h2(uint32_t a, uint32_t d) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) * __builtin_bit_cast(h2, d));
}
__device__ inline uint32_t residual_h2(uint32_t a, uint32_t d, uint32_t hi) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, d),
                                                                -__builtin_bit_cast(h2, hi)));
}
// Written per component: a loop over the vector's elements was compiled into
// element 0 replicated four times by this toolchain.
__device__ inline void scale_exact(const u4 a, const u4 d, u4& hi, u4& lo) {
  hi.x = mul_h2(a.x, d.x);
  hi.y = mul_h2(a.y, d.y);
  hi.z = mul_h2(a.z, d.z);
  hi.w = mul_h2(a.w, d.w);
  lo.x = residual_h2(a.x, d.x, hi.x);
  lo.y = residual_h2(a.y, d.y, hi.y);
  lo.z = residual_h2(a.z, d.z, hi.z);
  lo.w = residual_h2(a.w, d.w, hi.w);
}

// ------------------------------------------------------------ tile loads
//
// A tile is 32 positions of one (sequence, KV head): two 16-position groups
// ("halves"), each inside one page since page sizes are multiples of 16.
// Where a half's rows live is wave-uniform: its block-table entry is read
// with a scalar load and the row address stays in scalar registers, so a
// lane's load address is that base plus a fixed per-lane offset.  The loads
// land in raw registers that nothing reads until the tile is staged or
// computed, so the next tile's loads stay in flight while the current one is
// computed.  A half past the chunk end, or whose table entry lies outside the
// pool, re-reads an in-bounds group and is masked.

struct Half {
  size_t row;   // first row of the group (pool or contiguous storage)
  bool live;    // inside the chunk, with a valid table entry
};

// Where a group's rows are found.  Rows in LDS: entry j is the first pool
// row of the 16-position group at k0 + 16 j for this workgroup's KV head
// (the row-address arithmetic done once per group before the loop), or -1
// when its block-table entry lies outside the pool; entries past the chunk
// end are 0 (in bounds, masked).  A tile reads both of its entries with one
// 8-byte LDS read, issued a tile ahead.  Otherwise (contiguous storage, the
// chunk's first tile, or chunks of more groups than the LDS list holds:
// kGrpCap, half that for three or more tokens) the row comes
// from the block table through the constant address space (scalar loads).
// Either way the values are wave-uniform and never wait behind tile loads.
typedef __attribute__((address_space(3))) const int lds_int;
constexpr int kGrpCap = 1024;

struct Pages {
  lds_int* grp;
  bool in_lds;
};

// Locates the 16-position group at pos0 (all arguments wave-uniform) from the
// block table.  `bad` is set for a group inside the chunk whose table entry
// is outside the pool.
__device__ inline Half locate(const DecodeParams& p, int s, int h, int pos0, int k0, int k1, bool& bad) {
  const bool in = pos0 < k1;
  const int pos = in ? pos0 : k0;
  Half r;
  if (p.bt == nullptr) {
    const size_t cap = static_cast<size_t>(p.bt_stride) * p.page_size;
    r.row = (static_cast<size_t>(s) * kKvHeads + h) * cap + pos;
    r.live = in;
    return r;
  }
  const int lp = pos / p.page_size;
  const int slot = pos - lp * p.page_size;
  const int phys = reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
      reinterpret_cast<uintptr_t>(p.bt))[static_cast<size_t>(s) * p.bt_stride + lp];
  const bool ok = static_cast<unsigned>(phys) < static_cast<unsigned>(p.n_pool_blocks);
  if (in && !ok) bad = true;
  r.row = ok ? (static_cast<size_t>(phys) * kKvHeads + h) * p.page_size + slot : 0;
  r.live = in && ok;
  return r;
}

// The LDS row entries of tile ti's two groups (read early; used by the next
// load of that tile).
__device__ inline i2 read_rows(const Pages& pg, int ti) {
  return pg.in_lds ? *reinterpret_cast<const __attribute__((address_space(3))) i2*>(pg.grp + 2 * ti) : i2{0, 0};
}

// The group at pos0 from its LDS entry e (wave-uniform after readfirstlane).
__device__ inline Half from_entry(int e, int pos0, int k1, bool& bad) {
  const bool in = pos0 < k1;
  const bool ok = e >= 0;
  if (in && !ok) bad = true;
  Half r;
  r.row = ok ? static_cast<size_t>(e) : 0;
  r.live = in && ok;
  return r;
}

// Raw registers of one tile.  K: lane (m, g) holds the code bytes of dims
// 8g..8g+7 of every block of key m, as aligned dwords (blocks that start
// 2 bytes off a dword boundary take one dword more and are funnel-shifted
// when used); K scales: the dwords holding the scales of blocks 2g and 2g+1;
// V: quant rows, lane (j, seg) holds bytes [seg * 4 kVw, +4 kVw) of row j
// (whole blocks, split into codes and scales when staged); 16-bit rows,
// load i brings rows 2i and 2i + 1 whole, lane l the 16 bytes at 16 (l % 32)
// of row 2i + l / 32, so each load covers two rows contiguously.  K and V
// may be of different types.
template <int KT, int VT>
struct Tile {
  // raw K dwords per half (Q4_0: both halves as 5 16-byte pieces in kp)
  static constexpr int kKr = (KT == kQ4_0) ? 1 : (KT == kQ8_0) ? 20 : 32;
  static constexpr int kKp = (KT == kQ4_0) ? 20 : 1;
  static constexpr int kVw = (VT == kQ4_0) ? 9 : (VT == kQ8_0) ? 17 : 32;    // raw V dwords per half
  uint32_t k[2][kKr];
  uint32_t kp[kKp];
  uint32_t ks[2][2];
  uint32_t v[2][kVw];
  bool live[2];
};

// Q4_0 K: the two 16-row groups (2 x 2304 bytes) as 288 16-byte pieces;
// piece e = 64 i + lane of load i is byte 16 e' of group e >= 144 (e' the
// index inside its group).  Lanes past piece 287 re-read a piece of group 1.
__device__ inline int kpiece_group(int e) { return e >= 144 ? 1 : 0; }
__device__ inline uint32_t kpiece_off(int e) { return 16u * static_cast<uint32_t>(e >= 288 ? e - 288 : e >= 144 ? e - 144 : e); }

// First raw K dword of block b.
template <int KT>
__device__ constexpr int kraw(int b) {
  if constexpr (KT == kQ4_0) return 3 * (b >> 1) + ((b & 1) ? 2 : 0);
  else if constexpr (KT == kQ8_0) return 5 * (b >> 1) + ((b & 1) ? 3 : 0);
  else return 4 * b;
}

__device__ inline uint32_t ld32(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint32_t*>(base + off);
}
__device__ inline u2a ld64(const uint8_t* base, uint32_t off) { return *reinterpret_cast<const u2a*>(base + off); }
__device__ inline u4a ld128(const uint8_t* base, uint32_t off) { return *reinterpret_cast<const u4a*>(base + off); }

// Issues the loads of the tile at tb.  Only loads: no instruction here reads
// a loaded register.
template <int KT, int VT>
__device__ inline void load_tile(const DecodeParams& p, const Pages& pg, i2 rows, int s, int h, int tb, int k0,
                                 int k1, Tile<KT, VT>& t, bool& bad) {
  using F = Fmt<KT>;
  using FV = Fmt<VT>;
  const int lane = threadIdx.x & 63;
  const uint32_t m = lane & 15, g = lane >> 4;
  const uint32_t j = lane >> 2, seg = lane & 3;
  const uint8_t* rk_half[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const Half hv = pg.in_lds ? from_entry(__builtin_amdgcn_readfirstlane(rows[hf]), tb + 16 * hf, k1, bad)
                              : locate(p, s, h, tb + 16 * hf, k0, k1, bad);
    t.live[hf] = hv.live;
    const uint8_t* rk = p.k + hv.row * F::kRow;
    const uint8_t* rv = p.v + hv.row * FV::kRow;
    rk_half[hf] = rk;
    if constexpr (F::kKStage) {
      // K of both halves is loaded below as contiguous pieces
    } else if constexpr (KT == kF16 || KT == kBF16) {
      const uint32_t o = m * F::kRow + 16 * g;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const u4a x = ld128(rk, o + 64 * b);
        t.k[hf][4 * b] = x[0]; t.k[hf][4 * b + 1] = x[1]; t.k[hf][4 * b + 2] = x[2]; t.k[hf][4 * b + 3] = x[3];
      }
    } else if constexpr (KT == kQ8_0) {
      const uint32_t o = m * F::kRow + 8 * g;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int i = kraw<KT>(b);
        if (b & 1) {                        // codes start on a dword boundary
          const u2a x = ld64(rk, o + 34 * b + 2);
          t.k[hf][i] = x[0]; t.k[hf][i + 1] = x[1];
        } else {                            // 2 bytes off: three dwords around them
          const u2a x = ld64(rk, o + 34 * b);
          t.k[hf][i] = x[0]; t.k[hf][i + 1] = x[1];
          t.k[hf][i + 2] = ld32(rk, o + 34 * b + 8);
        }
      }
      t.ks[hf][0] = ld32(rk, m * F::kRow + 68 * g);
      t.ks[hf][1] = ld32(rk, m * F::kRow + 68 * g + 32);
    }
    if constexpr (VT == kF16 || VT == kBF16) {
      const uint32_t o = (lane >> 5) * FV::kRow + 16 * (lane & 31);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u4a x = ld128(rv, o + 2 * i * FV::kRow);
        t.v[hf][4 * i] = x[0]; t.v[hf][4 * i + 1] = x[1]; t.v[hf][4 * i + 2] = x[2]; t.v[hf][4 * i + 3] = x[3];
      }
    } else {
      constexpr int W = Tile<KT, VT>::kVw;
      const uint32_t o = j * FV::kRow + (W * 4) * seg;
#pragma unroll
      for (int i = 0; i + 4 <= W; i += 4) {
        const u4a x = ld128(rv, o + 4 * i);
        t.v[hf][i] = x[0]; t.v[hf][i + 1] = x[1]; t.v[hf][i + 2] = x[2]; t.v[hf][i + 3] = x[3];
      }
      t.v[hf][W - 1] = ld32(rv, o + 4 * (W - 1));
    }
  }
  if constexpr (F::kKStage) {
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int e = 64 * i + lane;
      const u4a x = ld128(kpiece_group(e) ? rk_half[1] : rk_half[0], kpiece_off(e));
      t.kp[4 * i] = x[0]; t.kp[4 * i + 1] = x[1]; t.kp[4 * i + 2] = x[2]; t.kp[4 * i + 3] = x[3];
    }
  }
}

// K operand of block b of half hf: 8 dims of one key as f16 (codes exact).
template <int KT, int VT>
__device__ inline u4 k_operand(const Tile<KT, VT>& t, const uint8_t* wk, int hf, int b) {
  const int i = kraw<KT>(b);
  if constexpr (KT == kQ4_0) {
    // raw row 16 hf + m in LDS: the 4 code bytes of dims 8g..8g+7 of block b
    // (2 bytes off a dword boundary for even b: two aligned dwords, shifted)
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
    const uint8_t* r = wk + Fmt<KT>::kKRaw + (16 * hf + m) * Fmt<KT>::kRow + 18 * b + 4 * g;
    uint32_t x;
    if (b & 1) {
      x = *reinterpret_cast<const uint32_t*>(r + 2);
    } else {
      const uint32_t lo = *reinterpret_cast<const uint32_t*>(r), hi = *reinterpret_cast<const uint32_t*>(r + 4);
      x = funnel16(lo, hi);
    }
    (void)i;
    (void)t;
    return q4_operand<true>(x);
  } else if constexpr (KT == kQ8_0) {
    if (b & 1) return q8_operand(t.k[hf][i], t.k[hf][i + 1]);
    return q8_operand(funnel16(t.k[hf][i], t.k[hf][i + 1]), funnel16(t.k[hf][i + 1], t.k[hf][i + 2]));
  } else {
    return u4{t.k[hf][i], t.k[hf][i + 1], t.k[hf][i + 2], t.k[hf][i + 3]};
  }
}

// Writes the tile's V rows into the V buffer `w` (quant V: codes and f16
// scales) and, for quant K, the K scales (f32) and key bias into the K area
// `wk`.  Keys at or past k1 are written as zeros.
template <int KT, int VT>
__device__ inline void stage_tile(uint8_t* w, uint8_t* wk, const Tile<KT, VT>& t, int tb, int k1) {
  using F = Fmt<KT>;
  using FV = Fmt<VT>;
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  const int j = lane >> 2, seg = lane & 3;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int key = 16 * hf + j;
    const bool valid = t.live[hf] && (tb + key < k1);
    if constexpr (VT == kF16 || VT == kBF16) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kr = 16 * hf + 2 * i + (lane >> 5);          // row of this lane's piece in load i
        u4 x = {t.v[hf][4 * i], t.v[hf][4 * i + 1], t.v[hf][4 * i + 2], t.v[hf][4 * i + 3]};
        if (!(t.live[hf] && tb + kr < k1)) x = u4{0, 0, 0, 0};
        *reinterpret_cast<u4*>(w + kr * FV::kVks + 16 * (lane & 31)) = x;
      }
    } else {
      float* vsc = reinterpret_cast<float*>(w + FV::kVtile);             // V scales: [8 blocks][4 groups][8] fp16
      const uint32_t* v = t.v[hf];
      u4 c0, c1, c2 = {0, 0, 0, 0}, c3 = {0, 0, 0, 0};
      uint32_t sa, sb;
      if constexpr (VT == kQ4_0) {
        c0 = u4{funnel16(v[0], v[1]), funnel16(v[1], v[2]), funnel16(v[2], v[3]), funnel16(v[3], v[4])};
        c1 = u4{v[5], v[6], v[7], v[8]};
        sa = v[0] & 0xFFFFu;
        sb = v[4] >> 16;
      } else {
        c0 = u4{funnel16(v[0], v[1]), funnel16(v[1], v[2]), funnel16(v[2], v[3]), funnel16(v[3], v[4])};
        c1 = u4{funnel16(v[4], v[5]), funnel16(v[5], v[6]), funnel16(v[6], v[7]), funnel16(v[7], v[8])};
        c2 = u4{v[9], v[10], v[11], v[12]};
        c3 = u4{v[13], v[14], v[15], v[16]};
        sa = v[0] & 0xFFFFu;
        sb = v[8] >> 16;
      }
      if (!valid) {
        c0 = c1 = c2 = c3 = u4{0, 0, 0, 0};
        sa = sb = 0u;
      }
      uint8_t* row = w + key * FV::kVks;
      if constexpr (VT == kQ4_0) {
        *reinterpret_cast<u4*>(row + 16 * (2 * seg)) = c0;
        *reinterpret_cast<u4*>(row + 16 * (2 * seg + 1)) = c1;
      } else {
        *reinterpret_cast<u4*>(row + 32 * (2 * seg)) = c0;
        *reinterpret_cast<u4*>(row + 32 * (2 * seg) + 16) = c1;
        *reinterpret_cast<u4*>(row + 32 * (2 * seg + 1)) = c2;
        *reinterpret_cast<u4*>(row + 32 * (2 * seg + 1) + 16) = c3;
      }
      // V scales as f16 in the element order of the V operand of lane group
      // g: key = 16 hf + 4 g + i is k-slot k = i + 4 hf of group g.
      {
        const int kk = (key & 3) + 4 * (key >> 4), gg = (key >> 2) & 3;
        int pos;
        if constexpr (VT == kQ4_0) pos = (kk & 3) * 2 + (kk >> 2);                 // pairs (0,4)(1,5)(2,6)(3,7)
        else pos = (kk < 4) ? (kk & 1) * 2 + (kk >> 1) : 4 + ((kk - 4) & 1) * 2 + ((kk - 4) >> 1);  // (0,2)(1,3)(4,6)(5,7)
        uint16_t* vh = reinterpret_cast<uint16_t*>(vsc);
        vh[((2 * seg) * 4 + gg) * 8 + pos] = static_cast<uint16_t>(sa);        // fp16 bits as stored
        vh[((2 * seg + 1) * 4 + gg) * 8 + pos] = static_cast<uint16_t>(sb);
      }
    }
    if constexpr (F::kQuant) {
      if constexpr (!F::kKStage) {
        // K scales: lane (m, g) holds blocks 2g, 2g+1 of key m of this half;
        // zero for keys that are not visible, so their codes give 0, not NaN
        float* ksc = reinterpret_cast<float*>(wk + F::kKScale);          // [2 halves][8 blocks][16 keys]
        float ka = half_bits(t.ks[hf][0] & 0xFFFFu), kb = half_bits(t.ks[hf][1] >> 16);
        if (!t.live[hf] || tb + 16 * hf + m >= k1) ka = kb = 0.f;
        ksc[(hf * 8 + 2 * g) * 16 + m] = ka;
        ksc[(hf * 8 + 2 * g + 1) * 16 + m] = kb;
      }
      if (seg == 0) {
        float* bias = reinterpret_cast<float*>(wk + F::kKBias);
        bias[hf * 16 + j] = valid ? 0.f : kNegInf;
      }
    }
  }
  if constexpr (F::kKStage) {
    // raw K rows of both halves: piece e at byte 16 e
    uint8_t* kr = wk + F::kKRaw;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int e = 64 * i + lane;
      if (e < 288) *reinterpret_cast<u4*>(kr + 16 * e) = u4{t.kp[4 * i], t.kp[4 * i + 1], t.kp[4 * i + 2], t.kp[4 * i + 3]};
    }
    wave_lds_sync();
    // K scales as f32 [half][block][16 keys]: lane l writes keys 4 (l % 4) ..
    // +3 of block (l / 4) % 8 of half l / 32
    const int hf = lane >> 5, b = (lane >> 2) & 7, m0 = 4 * (lane & 3);
    f4 d;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      d[i] = half_bits(*reinterpret_cast<const uint16_t*>(kr + (16 * hf + m0 + i) * F::kRow + 18 * b));
    // zero for keys that are not visible (a select on live: t stays in
    // registers); a tile inside the chunk with both halves live skips it
    if (!(t.live[0] && t.live[1] && tb + 32 <= k1)) {
      const bool lv = hf ? t.live[1] : t.live[0];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!lv || tb + 16 * hf + m0 + i >= k1) d[i] = 0.f;
    }
    *reinterpret_cast<f4*>(wk + F::kKScale + ((hf * 8 + b) * 16 + m0) * 4) = d;
  }
}

// Key of k-slot k (0..7) of lane group g in a 32-key tile: the layout of the
// QK result (lane (r, g) holds keys 4g..4g+3 of each 16-key half).
__device__ inline int sigma(int g, int k) { return (k < 4) ? 4 * g + k : 16 + 4 * g + (k - 4); }

// Query-row columns of the 16-wide B tiles: tile nt holds rows 16 nt ..
// 16 nt + 15, the hi and lo halves of q (and of the weights) in separate
// MFMAs.  A last tile of at most 8 rows (one, three, four or six tokens) is
// packed instead: lane n < 8 carries the hi part of row 16 nt + n, lane
// n + 8 the lo part of the same row, one MFMA takes both, and the two
// partial results are added across lanes n, n ^ 8.
template <int T>
struct Cols {
  static constexpr int R = 6 * T;
  static constexpr int NT = (R + 15) / 16;
  static constexpr bool kPackLast = (R - 16 * (NT - 1)) <= 8;
  static constexpr bool packed(int nt) { return kPackLast && nt == NT - 1; }
  // q operand tiles per 32-dim block in LDS: two per tile, one if packed
  static constexpr int kQParts = 2 * (NT - 1) + (kPackLast ? 1 : 2);
  // query row of column n of tile nt
  static constexpr int row(int nt, int n) { return 16 * nt + (packed(nt) ? (n & 7) : n); }
};

// Source of the QK^T B operands: an LDS copy laid out per (tile, part,
// block) as 64 lanes x 16 bytes, so each operand is one conflict-free
// 16-byte read per lane.
template <int T>
struct QSrc {
  const uint8_t* base;
  __device__ inline u4 get(int nt, int part, int b) const {
    return *reinterpret_cast<const u4*>(base + ((nt * 2 + part) * 8 + b) * 1024 + (threadIdx.x & 63) * 16);
  }
};

// QK^T of one tile: sacc[nt][hf] = S^T of half hf (lane (n, g): keys
// 4g..4g+3 of the half, column n), from the tile's K and the K area `wk`.
// Quant K: the accumulators start at the key bias (-inf for keys that are
// not visible; their zeroed scales keep the products finite), so no
// per-value mask is needed for the chunk end.
template <int KT, int T>
__device__ inline void qk_init(const uint8_t* wk, f4 (&sacc)[Cols<T>::NT][2]) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    f4 init = f4{0.f, 0.f, 0.f, 0.f};
    if constexpr (Fmt<KT>::kQuant) init = *reinterpret_cast<const f4*>(wk + Fmt<KT>::kKBias + (hf * 16 + 4 * g) * 4);
#pragma unroll
    for (int nt = 0; nt < Cols<T>::NT; ++nt) sacc[nt][hf] = init;
  }
}

// Block b (32 dims) of QK^T, both halves.
template <int KT, int VT, int T>
__device__ inline void qk_block(int b, const Tile<KT, VT>& t, const uint8_t* wk, const QSrc<T>& qs,
                                f4 (&sacc)[Cols<T>::NT][2]) {
  using F = Fmt<KT>;
  using C = Cols<T>;
  constexpr int NT = C::NT;
  constexpr bool BF = F::kBf;
  const int g = (threadIdx.x & 63) >> 4;
  u4 qb[NT][2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    qb[nt][0] = qs.get(nt, 0, b);
    if (!C::packed(nt)) qb[nt][1] = qs.get(nt, 1, b);
  }
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const u4 a = k_operand<KT, VT>(t, wk, hf, b);
    if constexpr (F::kQuant) {
      const f4 dk = *reinterpret_cast<const f4*>(wk + F::kKScale + ((hf * 8 + b) * 16 + 4 * g) * 4);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f4 cb = mma(a, qb[nt][0], f4{0.f, 0.f, 0.f, 0.f}, false);
        if (!C::packed(nt)) cb = mma(a, qb[nt][1], cb, false);
        sacc[nt][hf] += dk * cb;       // per-key block scale on the exact-code product
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        sacc[nt][hf] = mma(a, qb[nt][0], sacc[nt][hf], BF);
        if (!C::packed(nt)) sacc[nt][hf] = mma(a, qb[nt][1], sacc[nt][hf], BF);
      }
    }
  }
}

template <int T>
__device__ inline void qk_finish(f4 (&sacc)[Cols<T>::NT][2]) {
  if constexpr (Cols<T>::kPackLast) {
    constexpr int nt = Cols<T>::NT - 1;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[nt][hf][i] += lane_xor8(sacc[nt][hf][i]);
  }
}

// QK^T of one tile: sacc[nt][hf] = S^T of half hf (lane (n, g): keys
// 4g..4g+3 of the half, column n), from the tile's K and the K area `wk`.
// Quant K: the accumulators start at the key bias (-inf for keys that are
// not visible; their zeroed scales keep the products finite), so no
// per-value mask is needed for the chunk end.
template <int KT, int VT, int T>
__device__ inline void qk_tile(const Tile<KT, VT>& t, const uint8_t* wk, const QSrc<T>& qs,
                               f4 (&sacc)[Cols<T>::NT][2]) {
  qk_init<KT, T>(wk, sacc);
#pragma unroll
  for (int b = 0; b < 8; ++b) qk_block<KT, VT, T>(b, t, wk, qs, sacc);
  qk_finish<T>(sacc);
}

// Online softmax (base 2) of one tile.  Updates the running base and sum,
// returns the factor alpha[nt] by which the output accumulators must be
// scaled (the caller applies it, after any PV still in flight for the base
// before), and the PV B operands: the weights of keys sigma(g, k) split hi
// + lo (one token: this lane's part), in the V operand's key order.
// Returns true if some alpha is not 1.
template <int KT, int VT, int T>
__device__ inline bool softmax_tile(const f4 (&sacc)[Cols<T>::NT][2], const Tile<KT, VT>& t, int tb, int k1,
                                    const int (&lim)[Cols<T>::NT], int lim_min, float (&m_run)[Cols<T>::NT],
                                    float (&l_run)[Cols<T>::NT], float (&alpha)[Cols<T>::NT],
                                    u4 (&bh)[Cols<T>::NT], u4 (&bl)[Cols<T>::NT]) {
  using F = Fmt<KT>;
  using C = Cols<T>;
  constexpr int NT = C::NT;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const bool lo_lane = (n & 8) != 0;      // packed case: this lane carries lo parts
  // Quant K needs a mask only where the causal limit of some row (more than
  // one token) falls inside the tile; other types also at the chunk end.
  const bool full = (F::kQuant || tb + 32 <= k1) && (T == 1 || tb + 31 <= lim_min);
  bool any = false;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float sv[8];
    float mx = kNegInf;
    // key 16 hf + 4 g + i is visible iff 16 hf + i <= rel
    const int rel = min(k1 - 1, lim[nt]) - (tb + 4 * g);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = sacc[nt][hf][i];
        if (!full) x = (t.live[hf] && 16 * hf + i <= rel) ? x : kNegInf;
        sv[4 * hf + i] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    // The exponent base m_run moves only when the tile max exceeds it by more
    // than 8 (weights stay below 2^8), so the accumulators are rescaled rarely.
    float al = 1.f;
    if (mx > m_run[nt] + 8.f) {
      const float mn = mx;
      al = (m_run[nt] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run[nt] - mn);
      m_run[nt] = mn;
    }
    alpha[nt] = al;
    any |= (al != 1.f);
    // exp2(-inf) is 0; only an all-masked history (base still -inf) needs a
    // finite stand-in base
    const float mb = (m_run[nt] == kNegInf) ? 0.f : m_run[nt];
    float p[8];
    float rs = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      p[k] = __builtin_amdgcn_exp2f(sv[k] - mb);
      rs += p[k];
    }
    rs = sum_xor16(rs);
    rs = sum_xor32(rs);
    l_run[nt] = l_run[nt] * al + rs;
    // PV B operand from the 8 weights, in the V operand's key order
    float x[8];
    if constexpr (VT == kQ4_0) {
      constexpr int pi[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = p[pi[e]];
    } else if constexpr (VT == kQ8_0) {
      constexpr int pi[8] = {0, 2, 1, 3, 4, 6, 5, 7};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = p[pi[e]];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = p[e];
    }
    if constexpr (Fmt<VT>::kBf) {
      split8(x, bh[nt], bl[nt], true);
      if (C::packed(nt)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) bh[nt][k] = lo_lane ? bl[nt][k] : bh[nt][k];
      }
    } else if (C::packed(nt)) {
      u4 h, l;
      split8_rtz(x, h, l, -1.f);
#pragma unroll
      for (int k = 0; k < 4; ++k) bh[nt][k] = lo_lane ? l[k] : h[k];   // this lane's part
    } else {
      split8_rtz(x, bh[nt], bl[nt], -1.f);
    }
  }
  return __ballot(any) != 0;
}

// Block b of O^T += V^T P^T from the V buffer `wv` (quant V; for 16-bit V
// the two M-tiles of dims [32 b, 32 b + 32)).  Quant V: the operand is
// (c - 8) * d_v split exactly into hi + lo f16 parts.
template <int VT, int T>
__device__ inline void pv_block(int b, const uint8_t* wv, const u4 (&bh)[Cols<T>::NT], const u4 (&bl)[Cols<T>::NT],
                                f4 (&o)[Cols<T>::NT][16]) {
  using F = Fmt<VT>;
  using C = Cols<T>;
  constexpr int NT = C::NT;
  constexpr bool BF = F::kBf;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  if constexpr (F::kQuant) {
    const _Float16* vh = reinterpret_cast<const _Float16*>(wv + F::kVtile);
    const u4 dv = *reinterpret_cast<const u4*>(vh + (b * 4 + g) * 8);
    if constexpr (VT == kQ4_0) {
      // source lane n supplies key sigma(g, n % 8), code bytes [8 (n / 8), +8) of block b
      const uint8_t* src = wv + sigma(g, n & 7) * F::kVks + 16 * b + 8 * (n >> 3);
      const i2 r = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i2*)(src));
      u4 ah[2], al[2];
      scale_exact(q4_operand<false>(static_cast<uint32_t>(r[0])), dv, ah[0], al[0]);
      scale_exact(q4_operand<false>(static_cast<uint32_t>(r[1])), dv, ah[1], al[1]);
#pragma unroll
      for (int hm = 0; hm < 2; ++hm) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f4& acc = o[nt][2 * b + hm];
          acc = mma(ah[hm], bh[nt], acc, false);
          acc = mma(al[hm], bh[nt], acc, false);
          if (!C::packed(nt)) acc = mma(ah[hm], bl[nt], acc, false);
        }
      }
    } else {
#pragma unroll
      for (int hm = 0; hm < 2; ++hm) {
        // source lane n supplies key sigma(g, n / 2), code bytes [16 hm + 8 (n % 2), +8)
        const uint8_t* src = wv + sigma(g, n >> 1) * F::kVks + 32 * b + 16 * hm + 8 * (n & 1);
        const i2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2*)(src));
        u4 ah, al;
        scale_exact(q8_operand(static_cast<uint32_t>(r[0]), static_cast<uint32_t>(r[1])), dv, ah, al);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f4& acc = o[nt][2 * b + hm];
          acc = mma(ah, bh[nt], acc, false);
          acc = mma(al, bh[nt], acc, false);
          if (!C::packed(nt)) acc = mma(ah, bl[nt], acc, false);
        }
      }
    }
  } else {
#pragma unroll
    for (int mt = 2 * b; mt < 2 * b + 2; ++mt) {
      // source lane n supplies key sigma(g, n / 4) (then sigma(g, 4 + n / 4)), halves [16 mt + 4 (n % 4), +4)
      const uint8_t* s0 = wv + sigma(g, n >> 2) * F::kVks + 2 * (16 * mt + 4 * (n & 3));
      const uint8_t* s1 = wv + sigma(g, 4 + (n >> 2)) * F::kVks + 2 * (16 * mt + 4 * (n & 3));
      const s4 ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(s0));
      const s4 rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(s1));
      const u2 ua = __builtin_bit_cast(u2, ra), ub = __builtin_bit_cast(u2, rb);
      const u4 a = {ua[0], ua[1], ub[0], ub[1]};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        o[nt][mt] = mma(a, bh[nt], o[nt][mt], BF);
        if (!C::packed(nt)) o[nt][mt] = mma(a, bl[nt], o[nt][mt], BF);
      }
    }
  }
}

template <int VT, int T>
__device__ inline void pv_tile(const uint8_t* wv, const u4 (&bh)[Cols<T>::NT], const u4 (&bl)[Cols<T>::NT],
                               f4 (&o)[Cols<T>::NT][16]) {
#pragma unroll
  for (int b = 0; b < 8; ++b) pv_block<VT, T>(b, wv, bh, bl, o);
}

// QK^T of tile i interleaved block by block with the PV of the previous tile
// (independent work: in-order issue then finds one stream's instructions
// while the other waits on LDS or matrix-core results).
template <int KT, int VT, int T>
__device__ inline void qk_with_pv(const Tile<KT, VT>& t, const uint8_t* wk, const QSrc<T>& qs, f4 (&sacc)[Cols<T>::NT][2],
                                  const uint8_t* wv_prev, const u4 (&bh)[Cols<T>::NT], const u4 (&bl)[Cols<T>::NT],
                                  f4 (&o)[Cols<T>::NT][16]) {
  qk_init<KT, T>(wk, sacc);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    qk_block<KT, VT, T>(b, t, wk, qs, sacc);
    pv_block<VT, T>(b, wv_prev, bh, bl, o);
  }
  qk_finish<T>(sacc);
}

template <int T>
__device__ inline void rescale(f4 (&o)[Cols<T>::NT][16], const float (&alpha)[Cols<T>::NT]) {
#pragma unroll
  for (int nt = 0; nt < Cols<T>::NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) o[nt][mt] *= alpha[nt];
}

// One tile in sequence: QK^T, softmax, PV.
template <int KT, int VT, int T>
__device__ inline void compute_tile(const Tile<KT, VT>& t, const uint8_t* wv, const uint8_t* wk, int tb, int k1,
                                    const int (&lim)[Cols<T>::NT], int lim_min, const QSrc<T>& qs,
                                    f4 (&o)[Cols<T>::NT][16], float (&m_run)[Cols<T>::NT],
                                    float (&l_run)[Cols<T>::NT]) {
  constexpr int NT = Cols<T>::NT;
  f4 sacc[NT][2];
  qk_tile<KT, VT, T>(t, wk, qs, sacc);
  float alpha[NT];
  u4 bh[NT], bl[NT];
  if (softmax_tile<KT, VT, T>(sacc, t, tb, k1, lim, lim_min, m_run, l_run, alpha, bh, bl)) rescale<T>(o, alpha);
  pv_tile<VT, T>(wv, bh, bl, o);
}

// Output dim of accumulator element (M-tile mt, lane group g, element i).
template <int KT>
__device__ inline int out_dim(int mt, int g, int i) {
  const int m = 4 * g + i;
  if constexpr (KT == kQ4_0) return 32 * (mt >> 1) + 16 * (m & 1) + 8 * (mt & 1) + (m >> 1);
  return 16 * mt + m;
}

// Query operands (B of QK^T): q * scale * log2 e split hi + lo, element
// order matching the K operand's dim order of each type, written to LDS per
// (tile, part, block).  One token: lane n < 8 of a column group carries the
// hi part of row n, lane n + 8 the lo part (one tile, one part).  More
// tokens: hi and lo in separate parts.  Wave w builds blocks 2w and 2w+1.
// The loads are issued first (QLoad) and consumed later, so that the first
// tile's loads, issued in between, stay in flight while q is converted.
template <int T>
struct QLoad {
  float4 v[Cols<T>::NT][2][2];
};

// Rv: the query rows of the group's tokens (6 per token; fewer than 6T in
// a last group that holds fewer tokens than the kernel).  Other rows read
// row 0 and are zero.
template <int KT, int T>
__device__ inline void load_q(const DecodeParams& p, int s, int h, int tok0, int wave, int Rv, QLoad<T>& ql) {
  using C = Cols<T>;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    const int r = C::row(nt, n);
    const bool live = r < Rv;
    const float* qrow = p.q + ((static_cast<size_t>(s) * p.tok_total + tok0 + (live ? r / 6 : 0)) * kQHeads +
                               h * kGroup + (live ? r % 6 : 0)) * kHeadDim;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = 2 * wave + bb;
      if constexpr (KT == kQ4_0) {
        ql.v[nt][bb][0] = *reinterpret_cast<const float4*>(qrow + 32 * b + 4 * g);
        ql.v[nt][bb][1] = *reinterpret_cast<const float4*>(qrow + 32 * b + 16 + 4 * g);
      } else {
        ql.v[nt][bb][0] = *reinterpret_cast<const float4*>(qrow + 32 * b + 8 * g);
        ql.v[nt][bb][1] = *reinterpret_cast<const float4*>(qrow + 32 * b + 8 * g + 4);
      }
    }
  }
}

template <int KT, int T>
__device__ inline void build_q(const DecodeParams& p, const QLoad<T>& ql, int wave, int Rv, uint8_t* q_lds) {
  using C = Cols<T>;
  const int lane = threadIdx.x & 63, n = lane & 15;
#pragma unroll
  for (int nt = 0; nt < C::NT; ++nt) {
    const int r = C::row(nt, n);
    const bool live = r < Rv;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = 2 * wave + bb;
      float x[8];
      if constexpr (KT == kQ4_0) {
        const float4 lo = ql.v[nt][bb][0], hi = ql.v[nt][bb][1];
        x[0] = lo.x; x[1] = lo.z; x[2] = hi.x * 0.0625f; x[3] = hi.z * 0.0625f;
        x[4] = lo.y; x[5] = lo.w; x[6] = hi.y * 0.0625f; x[7] = hi.w * 0.0625f;
      } else {
        const float4 a = ql.v[nt][bb][0], bq = ql.v[nt][bb][1];
        if constexpr (KT == kQ8_0) {
          x[0] = a.x; x[1] = a.z; x[2] = a.y; x[3] = a.w; x[4] = bq.x; x[5] = bq.z; x[6] = bq.y; x[7] = bq.w;
        } else {
          x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = bq.x; x[5] = bq.y; x[6] = bq.z; x[7] = bq.w;
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = live ? x[i] * p.scale_log2 : 0.f;
      u4 hi, lo;
      split8(x, hi, lo, Fmt<KT>::kBf);
      if (C::packed(nt)) {
        *reinterpret_cast<u4*>(q_lds + ((nt * 2 + 0) * 8 + b) * 1024 + lane * 16) = (n & 8) ? lo : hi;
      } else {
        *reinterpret_cast<u4*>(q_lds + ((nt * 2 + 0) * 8 + b) * 1024 + lane * 16) = hi;
        *reinterpret_cast<u4*>(q_lds + ((nt * 2 + 1) * 8 + b) * 1024 + lane * 16) = lo;
      }
    }
  }
}

// Issue priority (set per tile in both loops below).  Two workgroups share
// each compute unit, and the hardware favours the older wave of a SIMD: with
// equal work the second workgroup to arrive finishes several microseconds
// after the first, and the kernel waits for it.  A wave takes priority 3, 2,
// 1, 0 by the share of its tiles still to do, so that one that falls behind
// its SIMD partner gets ahead in issue.  In the double-buffered loop the
// first workgroup of each unit (the first n_cu of the grid) stays at 0
// instead, which measured better there (the second one then catches up);
// in the single-buffer loop both follow their share.  Results do not depend
// on it.

// Register double-buffering of the next tile pays for the compact quant rows;
// the 16-bit rows use a single buffer (their loads are large enough that the
// other waves cover the latency).
template <int KT, int VT, int T>
constexpr bool kDoubleBuffer = (KT == kQ4_0 && VT == kQ4_0 && T == 1);

// Workgroups per compute unit the kernel is compiled for: two (8 waves per
// CU, at most 256 registers per lane) up to two tokens, and up to five
// tokens with quantized V, whose per-wave LDS buffers are small enough for
// two workgroups (with 16-bit V the buffers take one workgroup's share).
// Six or more tokens hold three 16-column output tiles (192 registers) and
// run one workgroup per CU.
template <int KT, int VT, int T>
constexpr int kMinWgs = (T <= 2 || (T <= 5 && Fmt<VT>::kQuant)) ? 2 : 1;

// kHost: instantiated for a host-planned launch (p.hp.on), whose plan
// lookup then starts without waiting on the flag.
template <int KT, int VT, int T, bool kHost>
__global__ __launch_bounds__(256, (kMinWgs<KT, VT, T>)) void split_mfma_kernel(DecodeParams p) {
  using F = Fmt<KT>;
  using FV = Fmt<VT>;
  using C = Cols<T>;
  constexpr int R = C::R;
  constexpr int NT = C::NT;
  // per wave: one V buffer, or two when PV runs one tile behind QK; then the K area
  constexpr int kWaveBytes = (kDoubleBuffer<KT, VT, T> ? 2 : 1) * FV::kVbuf + F::kKarea;
  // the combine, kRT rows at a time: [4 waves][kRT rows][256 + 4] floats
  // (the pad puts the rows a column group writes in different banks and
  // keeps them 16-byte aligned for vector writes).  One or two tokens take
  // their live rows in one pass; more tokens pass 8 rows at a time, which
  // keeps the buffer within the per-wave tile buffers it reuses.
  constexpr int kRedStride = kHeadDim + 4;
  constexpr int kRT = (R < 16) ? R : 8;
  constexpr int kPasses = (R + kRT - 1) / kRT;
  constexpr int kRed = 4 * kRT * kRedStride * 4;
  constexpr int kLds = (4 * kWaveBytes > kRed) ? 4 * kWaveBytes : kRed;
  constexpr int kQLds = C::kQParts * 8 * 1024;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[kQLds];
  // the group list: half as long (chunks up to 8192 positions) for three or
  // more tokens, whose LDS must leave room for a second workgroup; longer
  // chunks read the block table directly
  constexpr int kGrpN = (T <= 2) ? kGrpCap : kGrpCap / 2;
  __shared__ __attribute__((aligned(16))) int grp_lds[kGrpN];
  __shared__ float ml_lds[4][R][2];
  __shared__ float row_stat[2][R];                   // per row: 1 / sum of weights, log2-sum-exp
  __shared__ long long sh_sum[kPlanShared];
  __shared__ int sh_loc[4];
  __shared__ int sh_bad[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int cap = p.bt_stride * p.page_size;

  // Token groups: workgroup b takes item 8 (b / 8G) + b % 8 and group
  // (b / 8) % G, so the G groups of one chunk are dispatched 8 apart with the
  // same b % 8: on one XCD, sharing its L2 for the chunk's K/V, side by side
  const int bx = static_cast<int>(blockIdx.x);
  const int grp = (p.n_groups == 1) ? 0 : (bx / 8) % p.n_groups;
  const int item_id = (p.n_groups == 1) ? bx : (bx / (8 * p.n_groups)) * 8 + bx % 8;
  const int tok0 = p.tok0 + T * grp;                   // first token of this workgroup's rows
  const int jj = item_id / kKvHeads, h = item_id % kKvHeads;
  const PlanWG pl = plan_of<kHost ? 1 : 2>(p, cap, jj, -1, sh_sum, sh_loc);
  // every value that places loads is wave-uniform (scalar registers)
  const int chunk = __builtin_amdgcn_readfirstlane(pl.chunk);
  const int s = __builtin_amdgcn_readfirstlane(pl.s), c = __builtin_amdgcn_readfirstlane(pl.c);
  if (s < 0) return;
  if (!kHost && tid == 0 && c == 0 && h == 0 && tok0 == 0) {     // the plan, for the merge kernel
    int32_t* hdr = reinterpret_cast<int32_t*>(p.err);
    if (s < kHdrSeqs) hdr[2 + s] = jj;
    if (s == 0) hdr[1] = chunk;
  }
  const int L = kHost ? pl.len : __builtin_amdgcn_readfirstlane(p.seq_lens[s]);
  const int nc = n_chunks_of(L, cap, chunk);
  // this chunk's partial rows in the workspace
  const size_t part =
      (static_cast<size_t>(tok0 / 8) * p.part_items + static_cast<size_t>(pl.item) * kKvHeads + h) * p.part_rows +
      6 * (tok0 % 8);
  const size_t orow = static_cast<size_t>(s) * p.tok_total + tok0;   // output row of token 0 of the group
  // rows of the group's tokens: a last group may hold fewer tokens than the
  // kernel (matrix-core launches cover every token in whole groups); the
  // rows past them are computed on a zero query and never written
  const int Rv = 6 * min(T, p.tok_total - tok0);

  if (!len_ok(L, cap)) {   // corrupt length: NaN rows, nothing read
    const float nan = __builtin_nanf("");
    for (int i = tid; i < Rv * kHeadDim; i += kThreads) {
      const int r = i / kHeadDim, d = i % kHeadDim, t = r / 6, gq = r % 6;
      p.out[((orow + t) * kQHeads + h * kGroup + gq) * kHeadDim + d] = nan;
    }
    if (p.lse_out && tid < Rv) p.lse_out[(orow + tid / 6) * kQHeads + h * kGroup + tid % 6] = nan;
    if (tid == 0) atomicOr(p.err, 2u);
    return;
  }
  // token t of the group sits at position L - tok_total + tok0 + t and sees
  // the positions up to it; keys past the group's last token are skipped
  const int lim_base = L - p.tok_total + tok0;
  const int k0 = c * chunk;
  const int k1 = max(k0, min(min(L, k0 + chunk), lim_base + T));

  QSrc<T> qs;
  qs.base = q_lds;
  int lim[NT];
  const int lim_min = lim_base;                        // the first token's limit: every row sees <= lim_min
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = C::row(nt, n);                       // query row of this lane's column
    lim[nt] = lim_base + r / 6;                        // its token sees positions <= lim
  }

  f4 o[NT][16];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = kNegInf;
    l_run[nt] = 0.f;
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) o[nt][mt] = f4{0.f, 0.f, 0.f, 0.f};
  }

  uint8_t* wl = lds + wave * kWaveBytes;
  bool bad = false;
  const int n_tiles = (k1 > k0) ? (k1 - k0 + 31) / 32 : 0;

  // The rows of the chunk's 16-position groups go to LDS (read there once the
  // barrier below has passed); the first tile, loaded before it, reads the
  // table itself.  The table entries are loaded here and turned into rows
  // and written to LDS once q and the first tile are in flight as well
  // (loads return in order, so the writes wait for the table alone).  Row
  // indices are int32: pools of fewer than 2^31 rows per KV-head set.
  Pages pg{(lds_int*)(grp_lds), false};
  const int n_grp = 2 * n_tiles;                        // the tiles' groups (the last may lie past k1)
  const bool grp_fits = p.bt != nullptr && n_grp <= kGrpN &&
                        static_cast<long long>(p.n_pool_blocks) * kKvHeads * p.page_size < (1ll << 31);
  constexpr int kGrpPer = kGrpN / kThreads;
  int grp_v[kGrpPer];
  auto page_of = [&](int pos) { return (p.page_shift >= 0) ? (pos >> p.page_shift) : pos / p.page_size; };
  if (grp_fits) {
#pragma unroll
    for (int k = 0; k < kGrpPer; ++k) {
      const int j = tid + kThreads * k;
      const int pos = k0 + 16 * j;
      if (j < n_grp && pos < k1) grp_v[k] = p.bt[static_cast<size_t>(s) * p.bt_stride + page_of(pos)];
    }
  }
  auto stage_rows = [&]() {
    if (grp_fits) {
#pragma unroll
      for (int k = 0; k < kGrpPer; ++k) {
        const int j = tid + kThreads * k;
        const int pos = k0 + 16 * j;
        if (j < n_grp) {
          int row = 0;                                    // past the chunk: in bounds, masked
          if (pos < k1) {
            const int e = grp_v[k], lp = page_of(pos);
            row = (static_cast<unsigned>(e) < static_cast<unsigned>(p.n_pool_blocks))
                      ? (e * kKvHeads + h) * p.page_size + (pos - lp * p.page_size)
                      : -1;
          }
          grp_lds[j] = row;
        }
      }
    }
  };
  // issue priority 3, 2, 1, 0 by the quarter of this wave's tiles still to
  // do (it drops after own tile k = ((4 - j) total - 1) / 4, j = 3, 2, 1);
  // with double buffering the first workgroup of a unit stays at 0.  Only
  // when the grid is one round of resident workgroups: with more rounds, a
  // workgroup that finishes early makes room for the next one.
  const int my_total = (n_tiles - wave + 3) / 4;
  const int kq3 = (my_total - 1) >> 2, kq2 = (2 * my_total - 1) >> 2, kq1 = (3 * my_total - 1) >> 2;
  const bool one_round = p.max_items <= p.plan_slots;
  const bool follow = !kDoubleBuffer<KT, VT, T> || static_cast<int>(blockIdx.x) >= p.n_cu;
  auto set_prio = [&](int k) {                          // k: own index of the tile about to be staged
    if (!one_round) return;
    const int q = follow ? (k <= kq1) + (k <= kq2) + (k <= kq3) : 0;
    if (q >= 3) __builtin_amdgcn_s_setprio(3);
    else if (q == 2) __builtin_amdgcn_s_setprio(2);
    else if (q == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  };
  if constexpr (kDoubleBuffer<KT, VT, T>) {
    // Registers hold the next tile's loads while the current one is worked
    // on, and PV runs one tile behind: while tile i is staged, its QK^T and
    // softmax computed, the PV of tile i-4 (this wave's previous) runs from
    // the other V buffer, giving the scheduler two independent streams.
    // The output is rescaled for tile i's base only after that PV.
    uint8_t* wk = wl + 2 * FV::kVbuf;
    Tile<KT, VT> ta, tb2;
    int ti = wave;
    int kown = 1;
    QLoad<T> ql;
    i2 nrows = {0, 0};                    // LDS entries of this wave's next tile to load
    load_q<KT, T>(p, s, h, tok0, wave, Rv, ql);
    if (ti < n_tiles) load_tile<KT, VT>(p, pg, nrows, s, h, k0 + 32 * ti, k0, k1, ta, bad);
    stage_rows();
    build_q<KT, T>(p, ql, wave, Rv, q_lds);
    __syncthreads();
    pg.in_lds = grp_fits;
    if (ti + 4 < n_tiles) nrows = read_rows(pg, ti + 4);
    if (ti < n_tiles) {
      u4 bh[NT], bl[NT];                  // PV operands of the previous tile
      float alpha[NT];
      f4 sacc[NT][2];
      int vb = 0;                         // V buffer of the current tile
      // first tile: no PV behind it yet
      stage_tile<KT, VT>(wl, wk, ta, k0 + 32 * ti, k1);
      wave_lds_sync();
      if (ti + 4 < n_tiles) {
        load_tile<KT, VT>(p, pg, nrows, s, h, k0 + 32 * (ti + 4), k0, k1, tb2, bad);
        if (ti + 8 < n_tiles) nrows = read_rows(pg, ti + 8);
      }
      qk_tile<KT, VT, T>(ta, wk, qs, sacc);
      softmax_tile<KT, VT, T>(sacc, ta, k0 + 32 * ti, k1, lim, lim_min, m_run, l_run, alpha, bh, bl);
      wave_lds_sync();
      ti += 4;
      vb = 1;
      while (ti < n_tiles) {
        set_prio(kown++);
        stage_tile<KT, VT>(wl + vb * FV::kVbuf, wk, tb2, k0 + 32 * ti, k1);
        wave_lds_sync();
        if (ti + 4 < n_tiles) {
          load_tile<KT, VT>(p, pg, nrows, s, h, k0 + 32 * (ti + 4), k0, k1, ta, bad);
          if (ti + 8 < n_tiles) nrows = read_rows(pg, ti + 8);
        }
        qk_with_pv<KT, VT, T>(tb2, wk, qs, sacc, wl + (vb ^ 1) * FV::kVbuf, bh, bl, o);
        if (softmax_tile<KT, VT, T>(sacc, tb2, k0 + 32 * ti, k1, lim, lim_min, m_run, l_run, alpha, bh, bl))
          rescale<T>(o, alpha);
        wave_lds_sync();
        ti += 4;
        vb ^= 1;
        if (ti >= n_tiles) break;
        set_prio(kown++);
        stage_tile<KT, VT>(wl + vb * FV::kVbuf, wk, ta, k0 + 32 * ti, k1);
        wave_lds_sync();
        if (ti + 4 < n_tiles) {
          load_tile<KT, VT>(p, pg, nrows, s, h, k0 + 32 * (ti + 4), k0, k1, tb2, bad);
          if (ti + 8 < n_tiles) nrows = read_rows(pg, ti + 8);
        }
        qk_with_pv<KT, VT, T>(ta, wk, qs, sacc, wl + (vb ^ 1) * FV::kVbuf, bh, bl, o);
        if (softmax_tile<KT, VT, T>(sacc, ta, k0 + 32 * ti, k1, lim, lim_min, m_run, l_run, alpha, bh, bl))
          rescale<T>(o, alpha);
        wave_lds_sync();
        ti += 4;
        vb ^= 1;
      }
      pv_tile<VT, T>(wl + (vb ^ 1) * FV::kVbuf, bh, bl, o);   // the last tile's PV
    }
  } else {
    uint8_t* wk = wl + FV::kVbuf;
    {
      QLoad<T> ql;
      load_q<KT, T>(p, s, h, tok0, wave, Rv, ql);
      stage_rows();
      build_q<KT, T>(p, ql, wave, Rv, q_lds);
    }
    __syncthreads();
    pg.in_lds = grp_fits;
    i2 nrows = (wave < n_tiles) ? read_rows(pg, wave) : i2{0, 0};
    int kown = 0;
    for (int ti = wave; ti < n_tiles; ti += 4) {
      set_prio(kown++);
      Tile<KT, VT> tt;
      load_tile<KT, VT>(p, pg, nrows, s, h, k0 + 32 * ti, k0, k1, tt, bad);
      if (ti + 4 < n_tiles) nrows = read_rows(pg, ti + 4);
      stage_tile<KT, VT>(wl, wk, tt, k0 + 32 * ti, k1);
      wave_lds_sync();
      compute_tile<KT, VT, T>(tt, wl, wk, k0 + 32 * ti, k1, lim, lim_min, qs, o, m_run, l_run);
      wave_lds_sync();
    }
  }
  if constexpr (C::kPackLast) {     // add the lo-part columns into the hi-part columns
#pragma unroll
    for (int mt = 0; mt < 16; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[NT - 1][mt][i] += lane_xor8(o[NT - 1][mt][i]);
  }

  __builtin_amdgcn_s_setprio(0);
  // ---- combine the 4 waves, write this chunk's rows, then merge
  __syncthreads();                       // every wave is done with its LDS tile region
  if (g == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = 16 * nt + n;
      if (r < R) {
        ml_lds[wave][r][0] = m_run[nt];
        ml_lds[wave][r][1] = l_run[nt];
      }
    }
  }
  if (lane == 0) sh_bad[wave] = __ballot(bad) ? 1 : 0;
  __syncthreads();
  // per-row statistics of the 4 waves' states, once per row (read after the
  // next barrier)
  if (tid < R) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ml_lds[w][tid][0]);
    float ltot = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = ml_lds[w][tid][0];
      ltot += (mw == kNegInf) ? 0.f : ml_lds[w][tid][1] * exp2f(mw - M);
    }
    row_stat[0][tid] = ltot > 0.f ? 1.f / ltot : 0.f;
    row_stat[1][tid] = ltot > 0.f ? M + __log2f(ltot) : kNegInf;
  }
  float* red = reinterpret_cast<float*>(lds);
  const bool any_bad = (sh_bad[0] | sh_bad[1] | sh_bad[2] | sh_bad[3]) != 0;
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int q = 0; q < kPasses; ++q) {
    if (q > 0) __syncthreads();                      // the previous pass's rows have been read
    const int nt = (q * kRT) >> 4;                   // the B tile holding this pass's rows
    const int r = 16 * nt + n;
    if (r < R && r >= q * kRT && r < q * kRT + kRT) {
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, ml_lds[w][r][0]);
      const float a = (m_run[nt] == kNegInf) ? 0.f : exp2f(m_run[nt] - M);
      float* dst = red + (wave * kRT + (r - q * kRT)) * kRedStride;
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) {
        const f4 v = o[nt][mt] * a;
        if constexpr (VT == kQ4_0) {    // elements 0, 2 and 1, 3 hold adjacent dims
          typedef float f2 __attribute__((ext_vector_type(2)));
          *reinterpret_cast<f2*>(dst + out_dim<VT>(mt, g, 0)) = f2{v[0], v[2]};
          *reinterpret_cast<f2*>(dst + out_dim<VT>(mt, g, 1)) = f2{v[1], v[3]};
        } else {                        // elements 0..3 hold dims 16 mt + 4 g ..
          *reinterpret_cast<f4*>(dst + out_dim<VT>(mt, g, 0)) = v;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRT; ++j) {
      const int rr = q * kRT + j;
      if (rr >= Rv) break;                            // rows of tokens past the call's last
      const int t = rr / 6, gq = rr % 6;
      const float sum = red[(0 * kRT + j) * kRedStride + tid] + red[(1 * kRT + j) * kRedStride + tid] +
                        red[(2 * kRT + j) * kRedStride + tid] + red[(3 * kRT + j) * kRedStride + tid];
      float val = sum * row_stat[0][rr];
      float lse2 = row_stat[1][rr];
      if (any_bad) {
        val = nan;
        lse2 = nan;
      }
      if (nc == 1) {
        p.out[((orow + t) * kQHeads + h * kGroup + gq) * kHeadDim + tid] = val;
        if (p.lse_out && tid == 0) p.lse_out[(orow + t) * kQHeads + h * kGroup + gq] = lse2 * kLn2;
      } else {
        p.part_o[(part + rr) * kHeadDim + tid] = val;
        if (tid == 0) p.part_lse[part + rr] = lse2;
      }
    }
  }
  if (any_bad && tid == 0) atomicOr(p.err, 1u);
}

template <int KT, int VT>
hipError_t launch_kvt(const DecodeParams& p, const SplitLaunch& l) {
  // with token groups, items in whole blocks of 8 (the padding workgroups
  // find no plan item and return)
  const unsigned items = static_cast<unsigned>(grid_items(p));
  const dim3 grid(p.n_groups == 1 ? items : (items + 7) / 8 * 8 * static_cast<unsigned>(p.n_groups));
  void* args[] = {const_cast<DecodeParams*>(&p)};
  const void* f = p.hp.on ? reinterpret_cast<const void*>(&split_mfma_kernel<KT, VT, PA_T, true>)
                          : reinterpret_cast<const void*>(&split_mfma_kernel<KT, VT, PA_T, false>);
  return hipExtLaunchKernel(f, grid, dim3(kThreads), args, 0, l.stream, l.start, l.stop, 0);
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

// Resident workgroups per compute unit (the runtime's occupancy query).
template <int KT, int VT>
int wgs_per_cu() {
  static const int n = [] {
    int r = 0;
    // both plan sources' instantiations: the smaller of the two
    int r2 = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&r, split_mfma_kernel<KT, VT, PA_T, false>, kThreads, 0) !=
            hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&r2, split_mfma_kernel<KT, VT, PA_T, true>, kThreads, 0) !=
            hipSuccess)
      r = r2 = 1;
    r = r < r2 ? r : r2;
    return r < 1 ? 1 : (r > 4 ? 4 : r);
  }();
  return n;
}

template <int KT>
int wgs_kt(int v_type) {
  switch (v_type) {
    case kF16: return wgs_per_cu<KT, kF16>();
    case kBF16: return wgs_per_cu<KT, kBF16>();
    case kQ8_0: return wgs_per_cu<KT, kQ8_0>();
    default: return wgs_per_cu<KT, kQ4_0>();
  }
}

}  // namespace

template <>
int split_mfma_wgs_t<PA_T>(int k_type, int v_type) {
  switch (k_type) {
    case kF16: return wgs_kt<kF16>(v_type);
    case kBF16: return wgs_kt<kBF16>(v_type);
    case kQ8_0: return wgs_kt<kQ8_0>(v_type);
    default: return wgs_kt<kQ4_0>(v_type);
  }
}

template <>
hipError_t launch_split_mfma_t<PA_T>(const DecodeParams& p, const SplitLaunch& l) {
  switch (p.k_type) {
    case kF16: return launch_kt<kF16>(p, l);
    case kBF16: return launch_kt<kBF16>(p, l);
    case kQ8_0: return launch_kt<kQ8_0>(p, l);
    case kQ4_0: return launch_kt<kQ4_0>(p, l);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
