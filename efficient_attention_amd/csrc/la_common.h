// la_common.h -- device helpers shared by the gfx950 linear-attention kernels.
//
// Conventions used by every kernel:
//  * wave64; a workgroup of 256 threads is 4 waves.
//  * bf16 is carried as raw 16-bit patterns packed two per 32-bit word (low half = lower
//    index).  Rounding fp32 -> bf16 is round-to-nearest-even (v_cvt_pk_bf16_f32).
//  * MFMA lane layouts (checked on gfx950 hardware):
//      v_mfma_f32_16x16x32_bf16: A lane l holds row l%16, k = 8*(l/16)+e (e < 8);
//                                B lane l holds column l%16, the same k; the 4 results of
//                                lane l are rows 4*(l/16)+r (r < 4) of column l%16.
//    A reduction index may be mapped to the 8 k-slots of a lane in any order, as long
//    as both operands use the same mapping; several kernels use that to feed an MFMA result
//    straight back in as an operand without moving data between lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// phi(x) = elu(x) + 1 with alpha = 1: x + 1 above zero, exp(x) at or below zero
// ("Efficient Transformers: Linear Attention and Flash Attention", section "Linear attention",
// feature map elu + 1).  Since e^x >= 1 + x everywhere, phi(x) = max(x + 1, e^min(x, 0)), and
// e^min(x, 0) = min(e^x, 1) is the exp instruction with its output clamp: four instructions,
// no compare.  exp is the hardware base-2 exponential of x*log2(e) (it may flush to zero
// below x = -87); maximum() propagates NaN.
__device__ __forceinline__ float phi(float x) {
  const float e = __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(x * kLog2e), 0.f, 1.f);
  return __builtin_elementwise_maximum(x + 1.f, e);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two fp32 -> packed bf16 pair (round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t phi_pair(uint32_t w) {
  return pack_bf16(phi(bf_lo(w)), phi(bf_hi(w)));
}

__device__ __forceinline__ u32x4 phi_bf16x8(u32x4 x) {
  u32x4 r;
  r.x = phi_pair(x.x);
  r.y = phi_pair(x.y);
  r.z = phi_pair(x.z);
  r.w = phi_pair(x.w);
  return r;
}

// Sum of the 8 bf16 values of a packed vector, in fp32.
__device__ __forceinline__ float sum_bf16x8(u32x4 x) {
  return ((bf_lo(x.x) + bf_hi(x.x)) + (bf_lo(x.y) + bf_hi(x.y))) +
         ((bf_lo(x.z) + bf_hi(x.z)) + (bf_lo(x.w) + bf_hi(x.w)));
}

// 8x8 transpose of 16-bit elements held as 8 rows of 8 (one u32x4 per row).
// out[e] = (row0[e], row1[e], ..., row7[e]).
__device__ __forceinline__ uint32_t pick(uint32_t w_even_row, uint32_t w_odd_row, int e) {
  // low half of result = element e of the even row, high half = element e of the odd row
  return (e & 1) ? __builtin_amdgcn_perm(w_odd_row, w_even_row, 0x07060302u)
                 : __builtin_amdgcn_perm(w_odd_row, w_even_row, 0x05040100u);
}

__device__ __forceinline__ uint32_t word(const u32x4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    out[e].x = pick(word(in[0], e >> 1), word(in[1], e >> 1), e);
    out[e].y = pick(word(in[2], e >> 1), word(in[3], e >> 1), e);
    out[e].z = pick(word(in[4], e >> 1), word(in[5], e >> 1), e);
    out[e].w = pick(word(in[6], e >> 1), word(in[7], e >> 1), e);
  }
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 products on the bf16 MFMA from two-term splits (after Henry, Tang and Heinecke,
// "Leveraging the bfloat16 Artificial Intelligence Datatype For Higher-Precision Computations",
// ARITH 2019): x = hi + lo + rest with hi the truncation of x to bf16 (|lo| < 2^-7 |x|) and lo
// the bf16 rounding of x - hi (|rest| <= 2^-16 |x|, either sign).  x y is taken as all four
// products hi_x hi_y + hi_x lo_y + lo_x hi_y + lo_x lo_y (mfma_split), each exact, accumulated
// in fp32: what is dropped is the rests, below 2^-15 |x y| and of either sign, so sums do not
// drift.  (Three terms, without lo_x lo_y, drop up to 2^-14 |x y| always with the sign of x y.)
// Truncation gives lo the sign of x, which keeps the IEEE class of a product that involves an
// infinity: lo of +-inf is a finite number of its sign (the residual of the largest finite
// value), lo of a finite x that bf16 holds exactly is x 2^-100 instead of zero (so inf * lo is
// inf, not NaN), and lo of zero is zero (so a row whose features are all zero still gives 0/0).
// A quiet NaN stays NaN in hi.
__device__ __forceinline__ float split_rest(float x) {
  const float xc = __builtin_amdgcn_fmed3f(x, -0x1.fffffep127f, 0x1.fffffep127f);
  const float r = xc - __uint_as_float(__float_as_uint(xc) & 0xffff0000u);
  return __builtin_fmaf(xc, 0x1p-100f, r);
}
// the truncated bf16 pair (a in the low half)
__device__ __forceinline__ uint32_t trunc_pair(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
__device__ __forceinline__ void split4(const f32x4& x, u32x2& hi, u32x2& lo) {
  hi.x = trunc_pair(x.x, x.y);
  hi.y = trunc_pair(x.z, x.w);
  lo.x = pack_bf16(split_rest(x.x), split_rest(x.y));
  lo.y = pack_bf16(split_rest(x.z), split_rest(x.w));
}
// hi and lo of 8 values (two f32x4) as 16x16x32 operands
__device__ __forceinline__ void split8(const f32x4& x0, const f32x4& x1, u32x4& hi, u32x4& lo) {
  u32x2 h0, l0, h1, l1;
  split4(x0, h0, l0);
  split4(x1, h1, l1);
  hi = u32x4{h0.x, h0.y, h1.x, h1.y};
  lo = u32x4{l0.x, l0.y, l1.x, l1.y};
}

// acc + x y for split operands x = (xh, xl), y = (yh, yl) of a 16x16x32 product, smallest
// terms first
__device__ __forceinline__ f32x4 mfma_split(u32x4 xh, u32x4 xl, u32x4 yh, u32x4 yl, f32x4 acc) {
  acc = mfma_bf16(xl, yl, acc);
  acc = mfma_bf16(xl, yh, acc);
  acc = mfma_bf16(xh, yl, acc);
  return mfma_bf16(xh, yh, acc);
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

__device__ __forceinline__ u32x4 zero_u4() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

// 16-byte global load / store
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Row load without control flow: a row at or beyond `end` reads row end-1 instead (always a
// valid address); the caller masks such rows where it uses them.  Keeping loads out of
// branches, and the masking away from the load, lets the compiler leave the load in flight
// until the data is really needed.
__device__ __forceinline__ u32x4 ld16_clamp(const uint16_t* base, int64_t row, int64_t end,
                                            int64_t ld, int col) {
  const int64_t r = row < end ? row : end - 1;
  return ld16(base + r * ld + col);
}
// The same as a non-temporal load, for inputs read once (measured faster for the d = 128 stage-1
// state sums and the chunked causal kernel than loads that allocate in the caches)
__device__ __forceinline__ u32x4 ld16_clamp_nt(const uint16_t* base, int64_t row, int64_t end,
                                               int64_t ld, int col) {
  const int64_t r = row < end ? row : end - 1;
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + r * ld + col));
}
// Row `row` of a tile whose first row is `tile` (a wave-uniform pointer), 16 bytes at column
// `col`, reading row `last` instead of any row beyond it: the per-lane part of the address is a
// small non-negative 32-bit offset, which the load adds to the uniform base itself.  A
// non-temporal load: its callers stream inputs that are read once (measured faster in the
// non-causal forward than loads that allocate in the caches).
__device__ __forceinline__ u32x4 ld16_row(const uint16_t* tile, int row, int last, int ld, int col) {
  const int r = row < last ? row : last;
  const uint32_t bytes = (uint32_t)(r * ld + col) * 2u;
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(tile) + bytes));
}

// First row and last valid row (relative, clamped to [0, rows - 1]) of a tile of `rows` rows
// starting at token t of a sequence whose valid rows end at t_end (exclusive, t_end > 0).  A tile
// wholly past the end reads row t_end - 1 only.
struct TileRows {
  int64_t first;
  int last;
};
__device__ __forceinline__ TileRows tile_rows(int64_t t, int64_t t_end, int rows) {
  TileRows tr;
  tr.first = t < t_end ? t : t_end - 1;
  const int64_t lim = t_end - 1 - tr.first;
  tr.last = lim < rows - 1 ? (int)lim : rows - 1;
  return tr;
}

__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// v, or zero when keep is false, without control flow.  A conditional expression here would
// compile to a branch around the work that produced v, with register copies of loaded data
// that make the compiler wait for every load in flight.
__device__ __forceinline__ u32x4 keep_if(u32x4 v, bool keep) {
  const uint32_t m = 0u - (uint32_t)keep;
  v.x &= m;
  v.y &= m;
  v.z &= m;
  v.w &= m;
  return v;
}

// Token-major ("transposed") LDS tile layout, [rows][T] bf16 with rows = features: element
// (a, j) sits at a*(T + 16) + (a / 8)*8 + j.  Two access patterns must be conflict-free on the
// 64 four-byte banks, 16 lanes of a 16-byte access at a time:
//   * MFMA operand reads: 16 consecutive rows, one column.  The row stride of T/2 + 8 dwords
//     (an odd multiple of 8, mod 64) puts rows u = 0..7 on banks 8u (permuted), and the extra
//     4 dwords after every 8 rows moves rows 8..15 onto the 4-bank groups in between;
//   * transposed writes: 16 rows spaced 8 apart, one column.  Eight rows of stride add a
//     multiple of 64 banks, so only the 4 dwords per 8-row group separate them: 16 distinct
//     4-bank groups.
template <int T>
__device__ __forceinline__ int tofs(int a, int j) {
  static_assert(((T / 2 + 8) / 8) % 2 == 1, "row stride must be an odd multiple of 8 dwords");
  return a * (T + 16) + (a >> 3) * 8 + j;
}
template <int ROWS, int T>
constexpr int tsize() { return ROWS * (T + 16) + ROWS; }

// LDS transpose read (ds_read_b64_tr_b16, gfx950; lane layout checked on hardware).  Within each
// group of 16 lanes, lane i receives element i % 4 of the four 16-bit values read by lane
// 4e + i / 4, for e = 0..3.  So when lane j of the group addresses T[R + j / 4][C0 + 4 (j % 4)] of a
// row-major tile T, lane i receives T[R + e][C0 + i]: four rows of one column.
// Element (row, col) of an unpadded bf16 tile [.][LEN] whose 16-byte pieces are permuted by the
// row: piece p of row r sits at p ^ (r & 15) (r & 7 on 128-byte rows).  Measured on gfx950
// (LDS bank-conflict counters): the 16-row operand read (ds_read_b128, lane = row l16, piece g)
// is conflict-free, and the MFMA-result write (ds_write_b64, lane = row l16, 8 bytes at column
// 4 g) is 2-way, against 4-way for the same write on rows padded by 32 bytes (read either way:
// conflict-free) and 2-way reads with a permutation of 8 rows on rows of 16 or more pieces.
template <int LEN>
__device__ __forceinline__ int pswz(int row, int col) {
  static_assert(LEN % 64 == 0, "rows of at least 8 pieces");
  constexpr int RM = LEN / 8 >= 16 ? 15 : 7;
  return row * LEN + ((((col >> 3) ^ (row & RM))) << 3) + (col & 7);
}

__device__ __forceinline__ u32x2 ld_tr16(const uint16_t* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// 16x16x32 MFMA operand whose reduction index runs over the rows of a row-major LDS tile T
// (leading dimension ld): lane l holds column col0 + l % 16 and, in k slot 4h + e, row
// row0 + 16h + 4(l / 16) + e.  The row order is the one in which an MFMA result holds its rows
// (two 16-row tiles, rows 4(l / 16) + r), so such a result can be the other operand directly.
// With a row stride of 8 (mod 64) dwords every half-wave reads 8 rows x 32 bytes, conflict-free.
__device__ __forceinline__ u32x4 ld_rows_operand(const uint16_t* T, int ld, int row0, int col0,
                                                 int l16, int g) {
  const uint16_t* p = T + (row0 + 4 * g + (l16 >> 2)) * ld + col0 + 4 * (l16 & 3);
  const u32x2 lo = ld_tr16(p), hi = ld_tr16(p + 16 * ld);
  u32x4 r;
  r.x = lo.x;
  r.y = lo.y;
  r.z = hi.x;
  r.w = hi.y;
  return r;
}

// Wave-level sum over the 4 lanes that share l % 16 (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float sum_over_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

}  // namespace la
