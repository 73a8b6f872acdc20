// la_favor.hip -- linear attention with the FAVOR+ feature map on gfx950: non-causal form
// (state sums, their reduction, the output) and the recurrent decode step.
//
// Feature map.  "Efficient Transformers: Linear Attention and Flash Attention" (section "Linear
// attention: reordering the matmuls, not shrinking them") names FAVOR+ (Choromanski et al.,
// "Rethinking Attention with Performers") as the non-negative feature map whose inner products
// approximate the softmax kernel; its positive random features are
//     phi(x) = exp(W x' - |x'|^2 / 2) / sqrt(m),   x' = scale * x,   W [m][d],
// and the attention is that of eq. Attention_i with this phi: out_i = phi(q_i)^T S / phi(q_i)^T z
// with S = sum_j phi(k_j) v_j^T (m x d) and z = sum_j phi(k_j).
//
// Ranges.  The exponents w.x' - |x'|^2/2 can lie far outside fp32's range of exp, so no phi is
// ever formed on its own scale:
//   * keys: a state is stored as (S, z) with a log-scale c (true state = exp(c) (S, z)); the
//     features of a tile enter as exp(u - c) with c the running maximum of the exponents u, and
//     when a tile raises the maximum the accumulated sums are multiplied by exp(c_old - c_new)
//     first.  Partial states of different token ranges are brought to their common maximum
//     before they are added.
//   * queries: phi(q) multiplies numerator and denominator alike, so any positive factor per
//     query cancels; the output kernels use exp(scale (w.q - max_i w_i.q)), every feature <= 1,
//     which also drops the |q'|^2/2 and 1/sqrt(m) factors.
// Both are exact rewritings of the same quotient (no term is dropped), not approximations.
//
// MFMA use.  The projection W x is a dense contraction over d and goes through
// v_mfma_f32_16x16x32_bf16 with W and x as bf16 operands (both are bf16 inputs: exact) and fp32
// accumulation; the features are rounded to bf16 as the operand of the next product, as phi(K)
// is in the elu + 1 kernels.  The result layout of the projection is arranged to be the operand
// layout of the next product (see la_common.h), so features never go through LDS.
#include <math.h>

#include <type_traits>

#include "la_common.h"
#include "la_kernels.h"

namespace la {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};
// the largest spread (natural-log units) between a chunk's key maxima and its state's scale for
// which the causal kernel evaluates the whole chunk on the state's scale
constexpr float kSameScale = 40.f;
// exp(a (u - m)) as one FMA and the base-2 exponential: al2 = a log2(e), ml2 = m a log2(e)
__device__ __forceinline__ float fexp_shift(float u, float al2, float ml2) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(u, al2, -ml2));
}

// Cross-lane steps on the vector ALU (no LDS round trip; lane layouts checked on gfx950):
// v_permlane16_swap of a value with itself returns the values of the even and of the odd 16-lane
// row of the lane's row pair, v_permlane32_swap those of the lower and upper 32 lanes, and the
// DPP row rotate / row shift move values within a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, 0xF, 0xF, false));
}
// maximum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the same column of the four rows)
__device__ __forceinline__ float max_over_groups(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = fmaxf(__int_as_float(p[0]), __int_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(q[0]), __int_as_float(q[1]));
}
// sum over the same four lanes, in the same order on every lane: (r0 + r1) + (r2 + r3)
__device__ __forceinline__ float sum_over_rows(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(p[0]) + __int_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(q[0]) + __int_as_float(q[1]);
}
// the value of lane l % 16 (row 0) on every lane of its column
__device__ __forceinline__ float from_row0(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  const auto q = __builtin_amdgcn_permlane32_swap(p[0], p[0], false, false);
  return __int_as_float(q[0]);
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0x128>(x, x));  // row_ror:8
  x = fmaxf(x, dpp<0x124>(x, x));  // row_ror:4
  x = fmaxf(x, dpp<0x122>(x, x));  // row_ror:2
  x = fmaxf(x, dpp<0x121>(x, x));  // row_ror:1
  return max_over_groups(x);
}
// inclusive prefix maximum over the lanes of a 16-lane row (row_shr:n; a lane with no source
// keeps its own value)
__device__ __forceinline__ float prefix_max16(float x) {
  x = fmaxf(x, dpp<0x111>(x, x));
  x = fmaxf(x, dpp<0x112>(x, x));
  x = fmaxf(x, dpp<0x114>(x, x));
  x = fmaxf(x, dpp<0x118>(x, x));
  return x;
}

// sum of squares of 8 bf16 values, in fp32, fixed order
// acc + the squares of 8 bf16 values, two products per packed dot instruction (each product is
// exact in fp32)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float sq2_bf16(uint32_t w, float acc) {
  const bf16x2_t x = __builtin_bit_cast(bf16x2_t, w);
  return __builtin_amdgcn_fdot2_f32_bf16(x, x, acc, false);
}
__device__ __forceinline__ float sumsq_bf16x8(u32x4 x, float acc = 0.f) {
  return sq2_bf16(x.w, sq2_bf16(x.z, sq2_bf16(x.y, sq2_bf16(x.x, acc))));
}

__device__ __forceinline__ u32x2 ld8(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }

// V tiles [rows][D] in LDS, 16-byte pieces permuted per row so that the transposed operand
// reads (ld_v_rows) hit distinct bank groups: row r's piece b sits at piece b ^ 2((r / (128/D)) %
// (D/16)).
template <int D>
__device__ __forceinline__ int vofs(int r, int c) {
  constexpr int VRL = 128 / D;
  return r * D + ((((c >> 3) ^ (2 * ((r / VRL) % (D / 16))))) << 3) + (c & 7);
}
// 16x16x32 operand with k over 32 rows of a V tile starting at row0, column col0 + l16: k slot
// 4h + e is row row0 + 16h + 4g + e (the row order of an MFMA result, two 16-row tiles)
template <int D>
__device__ __forceinline__ u32x4 ld_v_rows(const uint16_t* Vt, int row0, int col0, int l16, int g) {
  const uint16_t* p0 = Vt + vofs<D>(row0 + 4 * g + (l16 >> 2), col0 + 4 * (l16 & 3));
  const u32x2 lo = ld_tr16(p0), hi = ld_tr16(p0 + 16 * D);
  u32x4 r;
  r.x = lo.x;
  r.y = lo.y;
  r.z = hi.x;
  r.w = hi.y;
  return r;
}

// Feature relabelling used where features meet MFMA operands over the feature index: stored
// feature q = 32 j + 8 g + 4 h + r is feature p = 32 j + 16 h + 4 g + r.  An MFMA result lane
// (g, r) of feature tiles 2j and 2j + 1 holds the 4 + 4 features that are 8 consecutive stored
// ones, and a 16x16x32 operand over features takes 8 consecutive stored features per lane group
// (one 16-byte LDS read).
__device__ __forceinline__ int favor_p_of_q(int q) {
  return (q & ~31) + 16 * ((q >> 2) & 1) + 4 * ((q >> 3) & 3) + (q & 3);
}

// ================================================================ stage 1: state sums
// Waves per workgroup of the state sums: 16 (one feature tile each) for M = 256 at D = 64, so
// that four waves share a SIMD; 8 for M = 128 or 256 at D = 128; 4 for M = 64.
#define FAVOR_NW(D, M) ((M) >= 256 && (D) == 64 ? 16 : (M) >= 128 ? 8 : 4)
// One workgroup (NW waves) sums the features of one token slice:
// S_p = sum_j phi(k_j) v_j^T, z_p = sum_j phi(k_j), with log-scale c_p.  The slice streams
// through LDS in tiles of 64 tokens (128 with 16 waves, 32 at D = M = 128; double-buffered, one
// barrier per tile); wave w owns the 16 FT features from w M / NW:
//   U = K_tile W_w^T on MFMA (A = token rows of K from LDS, B = this wave's rows of W, held in
//       registers for the whole slice) -> lane holds u for feature l16 of each of its feature
//       tiles and tokens 16 tt + 4 g + r of the tile's token tiles tt;
//   u = (scale U - (scale^2 |k|^2 / 2 + ln(M) / 2)) log2(e) per token, i.e. the exponent in
//       base-2 units (one FMA per element); the wave's running maximum c_w;
//   S_w += 2^(u - c_w)^T V_tile and z_w += 2^(u - c_w)^T 1 on MFMA, the exp values packed to
//       bf16 as the A operand in the result's own layout (token tiles 2s, 2s + 1 form k-step s),
//       V read transposed from LDS in the same token order.
// At the end the waves' blocks are brought to the workgroup maximum and written, the log-scale
// converted back to natural-log units.
// At D = M = 128 the kernel fits 128 VGPRs, so two workgroups share a compute unit: 32-token
// tiles, the next tile's loads issued after the projection, and V operands read in two halves.
// That took the non-causal forward at d = m = 128 (128 heads of 65,536 tokens) from 1.93 to
// 1.86 ms; the other shapes keep 64-token tiles and the early loads, which measured 1-2% faster
// for them.
#define FAVOR_STATE_WIDE(D, M) ((D) == 128 && (M) == 128)
template <int D, int M>
__global__ __launch_bounds__(FAVOR_NW(D, M) * 64) __attribute__((amdgpu_waves_per_eu(FAVOR_STATE_WIDE(D, M) ? 4 : 1)))
void favor_kv_state(FavorStateArgs a) {
  constexpr int NW = FAVOR_NW(D, M);
  constexpr int NT = 64 * NW;
  constexpr bool kWide = FAVOR_STATE_WIDE(D, M);
  constexpr int T = NW == 16 ? 2 * kFavorTile : (kWide ? kFavorTile / 2 : kFavorTile);
  constexpr int TT = T / 16;        // token tiles per tile
  constexpr int LDK = D + 16;
  constexpr int KA = D / 32;        // k-steps of the projection
  constexpr int DC = D / 16;        // value-column tiles
  constexpr int FW = M / NW;        // features per wave
  constexpr int FT = FW / 16;       // feature tiles per wave
  constexpr int PPR = D / 8;        // 16-byte pieces per row
  constexpr int RP = T * PPR / NT;  // pieces per thread and tensor
  constexpr int64_t REC = favor_rec(D, M);
  static_assert(FT >= 1 && RP >= 1 && TT % 2 == 0, "shape");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][T * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][T * D];
  __shared__ __attribute__((aligned(16))) float kt[2][T];
  __shared__ float cw_sh[NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t grp = blockIdx.x / a.slices, sl = blockIdx.x % a.slices;
  const int64_t bh = grp / a.groups_per_head, gi = grp % a.groups_per_head;
  const int64_t gs = gi * a.group_len;
  const int64_t ge = gs + a.group_len < a.n ? gs + a.group_len : a.n;
  const int64_t t0 = gs + sl * a.slice_len;
  const int64_t t1 = t0 + a.slice_len < ge ? t0 + a.slice_len : ge;
  float* rec = a.partials + (int64_t)blockIdx.x * REC;
  const uint16_t* K = reinterpret_cast<const uint16_t*>(a.k) + bh * a.n * D;
  const uint16_t* V = reinterpret_cast<const uint16_t*>(a.v) + bh * a.n * D;
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.w);

  if (t0 >= t1) {  // an empty slice: the empty state
    for (int64_t e = tid; e < (int64_t)M * D + M; e += NT) rec[e] = 0.f;
    if (tid == 0) rec[(int64_t)M * D + M] = kNegInf;
    return;
  }

  const float s = a.scale;
  const float kconst = 0.5f * logf((float)M);  // ln(sqrt(M))
  const float hs2 = 0.5f * s * s;
  const float sl2 = s * kLog2e;  // exponents are carried in base-2 units inside this kernel

  // this wave's rows of W as B operands: column = feature, k = d
  u32x4 wr[FT][KA];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) wr[ft][ks] = ld16(W + (int64_t)(wave * FW + ft * 16 + l16) * D + ks * 32 + g * 8);

  auto prow = [&](int p) { return tid / PPR + p * (NT / PPR); };
  const int pcol = (tid % PPR) * 8;
  u32x4 kr[RP], vr[RP];
  auto load = [&](int64_t tt) {
#pragma unroll
    for (int p = 0; p < RP; ++p) {
      kr[p] = ld16_clamp(K, tt + prow(p), t1, D, pcol);
      vr[p] = ld16_clamp(V, tt + prow(p), t1, D, pcol);
    }
  };
  // tile to LDS; rows past the slice end get a zero V row and an exponent offset of +inf (so
  // u = -inf and exp(u - c) = 0)
  auto store = [&](int b, int64_t tt) {
#pragma unroll
    for (int p = 0; p < RP; ++p) {
      const int row = prow(p);
      const bool ok = tt + row < t1;
      st16(&Ks[b][row * LDK + pcol], kr[p]);
      st16(&Vs[b][vofs<D>(row, pcol)], keep_if(vr[p], ok));
      float ss = sumsq_bf16x8(kr[p]);
#pragma unroll
      for (int off = 1; off < PPR; off <<= 1) ss += __shfl_xor(ss, off);
      if (tid % PPR == 0) kt[b][row] = ok ? (hs2 * ss + kconst) * kLog2e : __builtin_huge_valf();
    }
  };

  f32x4 acc[FT][DC], accz[FT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    accz[ft] = zero4();
#pragma unroll
    for (int ct = 0; ct < DC; ++ct) acc[ft][ct] = zero4();
  }
  const uint32_t one2 = 0x3F803F80u;  // two bf16 ones
  u32x4 ones;                          // B operand with a column of ones (column 0)
  ones.x = ones.y = ones.z = ones.w = (l16 == 0) ? one2 : 0u;
  float cw = kNegInf;

  load(t0);
  store(0, t0);
  __syncthreads();
  int b = 0;
  for (int64_t tt = t0; tt < t1; tt += T, b ^= 1) {
    if constexpr (!kWide) load(tt + T);  // next tile (clamped rows past the end; stored but never counted)
    f32x4 u[FT][TT];
    float tmax = kNegInf;
#pragma unroll
    for (int ti = 0; ti < TT; ++ti) {
      u32x4 ka[KA];
#pragma unroll
      for (int ks = 0; ks < KA; ++ks) ka[ks] = ld16(&Ks[b][(ti * 16 + l16) * LDK + ks * 32 + g * 8]);
      const f32x4 ktv = *reinterpret_cast<const f32x4*>(&kt[b][ti * 16 + 4 * g]);
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        u[ft][ti] = zero4();
#pragma unroll
        for (int ks = 0; ks < KA; ++ks) u[ft][ti] = mfma_bf16(ka[ks], wr[ft][ks], u[ft][ti]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u[ft][ti][r] = __builtin_fmaf(sl2, u[ft][ti][r], -ktv[r]);
          tmax = fmaxf(tmax, u[ft][ti][r]);
        }
      }
    }
    if constexpr (kWide) load(tt + T);
    tmax = wave_max(tmax);
    if (tmax > cw) {  // wave-uniform: rescale what this wave has summed to the new maximum
      const float al = __builtin_amdgcn_exp2f(cw - tmax);
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        accz[ft] *= al;
#pragma unroll
        for (int ct = 0; ct < DC; ++ct) acc[ft][ct] *= al;
      }
      cw = tmax;
    }
    auto pack_exp = [&](const f32x4& u0, const f32x4& u1) {  // 2^(u - c_w) of two token tiles, bf16
      u32x4 r;
      r.x = pack_bf16(__builtin_amdgcn_exp2f(u0[0] - cw), __builtin_amdgcn_exp2f(u0[1] - cw));
      r.y = pack_bf16(__builtin_amdgcn_exp2f(u0[2] - cw), __builtin_amdgcn_exp2f(u0[3] - cw));
      r.z = pack_bf16(__builtin_amdgcn_exp2f(u1[0] - cw), __builtin_amdgcn_exp2f(u1[1] - cw));
      r.w = pack_bf16(__builtin_amdgcn_exp2f(u1[2] - cw), __builtin_amdgcn_exp2f(u1[3] - cw));
      return r;
    };
#pragma unroll
    for (int st = 0; st < TT / 2; ++st) {
      if constexpr (!kWide) {
        u32x4 bv[DC];
#pragma unroll
        for (int ct = 0; ct < DC; ++ct) bv[ct] = ld_v_rows<D>(Vs[b], st * 32, ct * 16, l16, g);
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
          const u32x4 af = pack_exp(u[ft][2 * st], u[ft][2 * st + 1]);
          accz[ft] = mfma_bf16(af, ones, accz[ft]);
#pragma unroll
          for (int ct = 0; ct < DC; ++ct) acc[ft][ct] = mfma_bf16(af, bv[ct], acc[ft][ct]);
        }
      } else {  // one feature tile per wave; V operands in two halves of the value columns
        static_assert(FT == 1 && DC % 2 == 0, "shape");
        constexpr int CG = DC / 2;
        u32x4 bv[CG];
#pragma unroll
        for (int c = 0; c < CG; ++c) bv[c] = ld_v_rows<D>(Vs[b], st * 32, c * 16, l16, g);
        const u32x4 af = pack_exp(u[0][2 * st], u[0][2 * st + 1]);
        accz[0] = mfma_bf16(af, ones, accz[0]);
#pragma unroll
        for (int c = 0; c < CG; ++c) acc[0][c] = mfma_bf16(af, bv[c], acc[0][c]);
#pragma unroll
        for (int c = 0; c < CG; ++c) bv[c] = ld_v_rows<D>(Vs[b], st * 32, (CG + c) * 16, l16, g);
#pragma unroll
        for (int c = 0; c < CG; ++c) acc[0][CG + c] = mfma_bf16(af, bv[c], acc[0][CG + c]);
      }
    }
    store(b ^ 1, tt + T);
    __syncthreads();
  }

  // common scale of the waves' blocks
  if (lane == 0) cw_sh[wave] = cw;
  __syncthreads();
  float cmax = kNegInf;
#pragma unroll
  for (int w = 0; w < NW; ++w) cmax = fmaxf(cmax, cw_sh[w]);
  const float be = cw == kNegInf ? 0.f : __builtin_amdgcn_exp2f(cw - cmax);
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    const int f0 = wave * FW + ft * 16 + 4 * g;
#pragma unroll
    for (int ct = 0; ct < DC; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) rec[(int64_t)(f0 + r) * D + ct * 16 + l16] = acc[ft][ct][r] * be;
    if (l16 == 0)
#pragma unroll
      for (int r = 0; r < 4; ++r) rec[(int64_t)M * D + f0 + r] = accz[ft][r] * be;
  }
  if (tid == 0) rec[(int64_t)M * D + M] = cmax * kLn2;  // the record's scale is in natural-log units
}

// ================================================================ stage 2: one state per group
// state = sum_p exp(c_p - c) (S_p, z_p) with c = max_p c_p, slices added in order.  Eight
// workgroups per group, each over an eighth of the record.
template <int D, int M>
__global__ __launch_bounds__(256) void favor_reduce(FavorReduceArgs a) {
  constexpr int64_t REC = favor_rec(D, M);
  constexpr int64_t BODY = (int64_t)M * D + M;  // multiple of 8
  constexpr int64_t PART = BODY / 8;
  constexpr int kMaxSlices = 64;
  __shared__ float fac[kMaxSlices];
  const int64_t grp = blockIdx.x / 8, part = blockIdx.x % 8;
  const float* P = a.partials + grp * a.slices * REC;
  float c = kNegInf;
  for (int64_t p = 0; p < a.slices; ++p) c = fmaxf(c, P[p * REC + BODY]);
  if (threadIdx.x < a.slices) {
    const float cp = P[threadIdx.x * REC + BODY];
    fac[threadIdx.x] = cp == kNegInf ? 0.f : fexp(cp - c);
  }
  __syncthreads();
  float* out = a.state + grp * REC;
  for (int64_t e = part * PART + threadIdx.x; e < (part + 1) * PART; e += 256) {
    float acc = 0.f;
    for (int64_t p = 0; p < a.slices; ++p) acc += fac[p] * P[p * REC + e];
    out[e] = acc;
  }
  if (part == 0 && threadIdx.x == 0) out[BODY] = c;
}

// ================================================================ non-causal output
// One workgroup (8 waves) per kFavorQueries queries of a head; a wave takes 16-query tiles, the
// next tile's query rows in flight while it computes the current one.  LDS (72 KB or less, so
// two workgroups share a compute unit), features in operand order (favor_p_of_q), every row's
// 16-byte pieces XOR-permuted by the row index (swz) so that 16 rows read at one column are
// conflict-free without padding: the head's state transposed, St[c][q] = bf16(S[p(q)][c]); a
// normaliser tile Zr with rows bf16(z) and bf16(z - bf16(z)) (rows 2..15 zero); W [M][D].  Per
// tile, outputs transposed:
//   U^T = W Q^T (A = rows of W, B = the lane's own query row from global memory): lane holds
//       features 16 ft + 4g + r of query l16;
//   f = exp(scale (U - max_f U)) packed to bf16 in the result layout: the B operand of the next
//       product, k slot e of lane group g = stored feature 32 j + 8 g + e;
//   out^T = St f (A = 16-byte rows of St), den = Zr f; out = out^T / den.

template <int D, int M>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) void favor_out(FavorOutArgs a) {
  constexpr int NT = 512;
  constexpr int QT = (int)kFavorQueries;
  constexpr int KA = D / 32;
  constexpr int DC = D / 16;
  constexpr int MT = M / 16;        // feature tiles
  constexpr int MJ = M / 32;        // k-steps over features
  constexpr int64_t REC = favor_rec(D, M);
  static_assert(D / 8 >= 8 && M / 8 >= 8, "the row permutation needs 8 pieces per row");

  __shared__ __attribute__((aligned(16))) uint16_t St[D * M];
  __shared__ __attribute__((aligned(16))) uint16_t Zr[16 * M];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[M * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  // all tiles of a head on one XCD (workgroups go to the 8 XCDs round-robin), so that its L2
  // serves the head's state to every tile
  const int64_t tiles = (a.n + QT - 1) / QT;
  int64_t bh, tile;
  if (a.bh % 8 == 0) {
    const int64_t x = blockIdx.x % 8, j = blockIdx.x / 8;
    bh = (j / tiles) * 8 + x;
    tile = j % tiles;
  } else {
    bh = blockIdx.x / tiles;
    tile = blockIdx.x % tiles;
  }
  const float* st = a.state + bh * REC;
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.w);
  const uint16_t* Q = reinterpret_cast<const uint16_t*>(a.q) + bh * a.n * D;
  uint16_t* O = reinterpret_cast<uint16_t*>(a.out) + bh * a.n * D;
  const int64_t qbase = tile * QT;

  // the first tile's query rows, before the set-up
  u32x4 qb[KA];
  int qt = wave;
#pragma unroll
  for (int ks = 0; ks < KA; ++ks) qb[ks] = ld16_clamp(Q, qbase + qt * 16 + l16, a.n, D, ks * 32 + g * 8);

  // St[c][q], stored features in pairs (q even: p(q + 1) = p(q) + 1); Zr; W.  Every load of the
  // set-up is issued before the first store, so the L2 latency is paid once.
  constexpr int SP = M * D / 2 / NT;   // feature pairs per thread
  constexpr int WP = M * D / 8 / NT;   // 16-byte pieces of W per thread
  float sv[SP][2];
  u32x4 wv[WP];
#pragma unroll
  for (int i = 0; i < SP; ++i) {
    const int e = tid + i * NT;
    const int pf = favor_p_of_q(2 * (e / D)), c = e % D;
    sv[i][0] = st[pf * D + c];
    sv[i][1] = st[(pf + 1) * D + c];
  }
  const float zq = tid < M ? st[M * D + favor_p_of_q(tid)] : 0.f;
#pragma unroll
  for (int i = 0; i < WP; ++i) {
    const int e = tid + i * NT;
    wv[i] = ld16(W + (e / (D / 8)) * D + (e % (D / 8)) * 8);
  }
#pragma unroll
  for (int i = 0; i < SP; ++i) {
    const int e = tid + i * NT;
    *reinterpret_cast<uint32_t*>(&St[pswz<M>(e % D, 2 * (e / D))]) = pack_bf16(sv[i][0], sv[i][1]);
  }
  for (int e = tid; e < 16 * M; e += NT) Zr[e] = 0;
#pragma unroll
  for (int i = 0; i < WP; ++i) {
    const int e = tid + i * NT;
    st16(&Ws[pswz<D>(e / (D / 8), (e % (D / 8)) * 8)], wv[i]);
  }
  __syncthreads();  // Zr cleared before its first two rows are written
  if (tid < M) {
    const __bf16 hi = (__bf16)zq;
    Zr[pswz<M>(0, tid)] = __builtin_bit_cast(uint16_t, hi);
    Zr[pswz<M>(1, tid)] = __builtin_bit_cast(uint16_t, (__bf16)(zq - (float)hi));
  }
  __syncthreads();

  const float s = a.scale;
  const float sl2 = s * kLog2e;
  for (; qt < QT / 16; qt += NT / 64) {
    const int64_t q0 = qbase + qt * 16;
    if (q0 >= a.n) break;
    u32x4 qn[KA];  // next tile's rows (clamped; unused past the end)
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) qn[ks] = ld16_clamp(Q, q0 + (NT / 64) * 16 + l16, a.n, D, ks * 32 + g * 8);
    f32x4 u[MT];
    float mq = kNegInf;
#pragma unroll
    for (int ft = 0; ft < MT; ++ft) {
      u[ft] = zero4();
#pragma unroll
      for (int ks = 0; ks < KA; ++ks) u[ft] = mfma_bf16(ld16(&Ws[pswz<D>(ft * 16 + l16, ks * 32 + g * 8)]), qb[ks], u[ft]);
#pragma unroll
      for (int r = 0; r < 4; ++r) mq = fmaxf(mq, u[ft][r]);
    }
    mq = max_over_groups(mq);
    const float mq_l2 = mq * sl2;
    u32x4 fq[MJ];
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
      fq[j].x = pack_bf16(fexp_shift(u[2 * j][0], sl2, mq_l2), fexp_shift(u[2 * j][1], sl2, mq_l2));
      fq[j].y = pack_bf16(fexp_shift(u[2 * j][2], sl2, mq_l2), fexp_shift(u[2 * j][3], sl2, mq_l2));
      fq[j].z = pack_bf16(fexp_shift(u[2 * j + 1][0], sl2, mq_l2), fexp_shift(u[2 * j + 1][1], sl2, mq_l2));
      fq[j].w = pack_bf16(fexp_shift(u[2 * j + 1][2], sl2, mq_l2), fexp_shift(u[2 * j + 1][3], sl2, mq_l2));
    }
    f32x4 acco[DC];
    f32x4 accd = zero4();
#pragma unroll
    for (int ct = 0; ct < DC; ++ct) acco[ct] = zero4();
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
#pragma unroll
      for (int ct = 0; ct < DC; ++ct)
        acco[ct] = mfma_bf16(ld16(&St[pswz<M>(ct * 16 + l16, 32 * j + 8 * g)]), fq[j], acco[ct]);
      accd = mfma_bf16(ld16(&Zr[pswz<M>(l16, 32 * j + 8 * g)]), fq[j], accd);
    }
    const float den = from_row0(accd[0] + accd[1]);
    const float inv = 1.0f / den;
    // lane rows g and g ^ 1 swap halves of a column-tile pair (v_permlane16_swap) so that a lane
    // holds 8 consecutive columns of one query: one 16-byte store
    const int64_t row = q0 + l16;
#pragma unroll
    for (int ct = 0; ct < DC; ct += 2) {
      const uint32_t ax = pack_bf16(acco[ct][0] * inv, acco[ct][1] * inv);
      const uint32_t ay = pack_bf16(acco[ct][2] * inv, acco[ct][3] * inv);
      const uint32_t bx = pack_bf16(acco[ct + 1][0] * inv, acco[ct + 1][1] * inv);
      const uint32_t by = pack_bf16(acco[ct + 1][2] * inv, acco[ct + 1][3] * inv);
      const auto sx = __builtin_amdgcn_permlane16_swap(ax, bx, false, false);
      const auto sy = __builtin_amdgcn_permlane16_swap(ay, by, false, false);
      u32x4 o;
      o.x = sx[0];
      o.y = sy[0];
      o.z = sx[1];
      o.w = sy[1];
      if (row < a.n) st16(O + row * D + (ct + (g & 1)) * 16 + 8 * (g >> 1), o);
    }
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) qb[ks] = qn[ks];
  }
}

// ================================================================ decode step
// One workgroup per head, in place on (S, z, c):
//   u_f = scale w_f.k - scale^2 |k|^2/2 - ln(M)/2,  c' = max(c, max_f u_f),  a = exp(c - c'),
//   S' = a S + exp(u - c') v^T,  z' = a z + exp(u - c'),
//   out = f^T S' / f^T z' with f = exp(scale (w.q - max_f w_f.q)).
// The projections are fp32 dot products of the bf16 rows of W (read through L2; W is shared by
// all heads) with k and q; the state update is a read-modify-write stream over S: each thread
// owns 4 adjacent columns and M / RG rows, loads them all first, and keeps a running column
// sum of f_a S'[a][c].  Sums are combined through LDS in a fixed order (bitwise reproducible).
template <int D, int M>
__global__ __launch_bounds__(256) void favor_decode(FavorDecodeArgs a) {
  constexpr int CG = D / 4;         // column groups of 4
  constexpr int RG = 256 / CG;      // row groups
  constexpr int RPT = M / RG;       // rows per thread
  __shared__ float qs[D], ks[D], vs[D];
  __shared__ float fk[M], fq[M];
  __shared__ float red[RG][D];
  __shared__ float wk[4], wmk[4], wmq[4], wd[4];  // per-wave partials (one array per reduction)

  const int64_t h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = tid % CG, rg = tid / CG;
  float* S = a.S + h * M * D;

  f32x4 sv[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r)  // non-temporal, as in decode_step_kernel: read once per step
    sv[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (int64_t)(rg + RG * r) * D + cg * 4));
  // the scale and z of the state, loaded with S (only this workgroup writes them, at the end)
  const float c_old = a.c[h];
  const float z_old = tid < M ? a.z[h * M + tid] : 0.f;

  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + h * D;
  const uint16_t* k = reinterpret_cast<const uint16_t*>(a.k) + h * D;
  const uint16_t* v = reinterpret_cast<const uint16_t*>(a.v) + h * D;
  float kk = 0.f;
  if (tid < D) {
    qs[tid] = __uint_as_float((uint32_t)q[tid] << 16);
    const float kv = __uint_as_float((uint32_t)k[tid] << 16);
    ks[tid] = kv;
    vs[tid] = __uint_as_float((uint32_t)v[tid] << 16);
    kk = kv * kv;
  }
  // |k|^2: wave sums in lane order, then the waves in order
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) kk += __shfl_xor(kk, off);
  if (lane == 0) wk[wave] = kk;
  __syncthreads();
  const float knorm = (wk[0] + wk[1]) + (wk[2] + wk[3]);
  const float s = a.scale;
  float uk = kNegInf, uq = kNegInf;
  if (tid < M) {
    const uint16_t* wrow = reinterpret_cast<const uint16_t*>(a.w) + (int64_t)tid * D;
    float dk = 0.f, dq = 0.f;
#pragma unroll
    for (int c0 = 0; c0 < D; c0 += 8) {
      const u32x4 w8 = ld16(wrow + c0);
      const float wv[8] = {bf_lo(w8.x), bf_hi(w8.x), bf_lo(w8.y), bf_hi(w8.y),
                           bf_lo(w8.z), bf_hi(w8.z), bf_lo(w8.w), bf_hi(w8.w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dk += wv[e] * ks[c0 + e];
        dq += wv[e] * qs[c0 + e];
      }
    }
    uk = s * dk - (0.5f * s * s * knorm + 0.5f * logf((float)M));
    uq = dq;
  }
  const float mk = wave_max(uk), mq = wave_max(uq);
  if (lane == 0) {
    wmk[wave] = mk;
    wmq[wave] = mq;
  }
  __syncthreads();
  const float umax = fmaxf(fmaxf(wmk[0], wmk[1]), fmaxf(wmk[2], wmk[3]));
  const float qmax = fmaxf(fmaxf(wmq[0], wmq[1]), fmaxf(wmq[2], wmq[3]));
  const float c_new = fmaxf(c_old, umax);
  const float al = c_old == kNegInf ? 0.f : fexp(c_old - c_new);
  float dpart = 0.f;
  if (tid < M) {
    const float ek = fexp(uk - c_new);
    const float eq = fexp(s * (uq - qmax));
    fk[tid] = ek;
    fq[tid] = eq;
    const float znew = al * z_old + ek;
    a.z[h * M + tid] = znew;
    dpart = eq * znew;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) dpart += __shfl_xor(dpart, off);
  if (lane == 0) wd[wave] = dpart;
  __syncthreads();  // fk, fq and wd written; every thread has read c
  if (tid == 0) a.c[h] = c_new;

  const f32x4 v4 = *reinterpret_cast<const f32x4*>(&vs[cg * 4]);
  f32x4 num = zero4();
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int row = rg + RG * r;
    const float ka = fk[row], qa = fq[row];
    sv[r] = sv[r] * al + ka * v4;
    // non-temporal, as in decode_step_kernel: not read again before the next step
    __builtin_nontemporal_store(sv[r], reinterpret_cast<f32x4*>(S + (int64_t)row * D + cg * 4));
    num += qa * sv[r];
  }
  *reinterpret_cast<f32x4*>(&red[rg][cg * 4]) = num;
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) acc += red[r][tid];
    const float den = (wd[0] + wd[1]) + (wd[2] + wd[3]);
    reinterpret_cast<__bf16*>(a.out)[h * D + tid] = (__bf16)(acc / den);
  }
}

// ================================================================ causal, chunked
// One workgroup (8 waves) walks one segment of one head in chunks of C = 64 tokens, like the
// elu + 1 chunked kernel (la_causal.hip): for the queries of a chunk
//   num = f(Q) S_prev + tril(f(Q) phi(K_c)^T) V_c,  den = f(Q) z_prev + tril(...) 1,
// then S += phi(K_c)^T V_c, z += phi(K_c)^T 1, with f(Q) the per-query-shifted features (the shift
// cancels in num / den).  Scales: the state is kept on a log-scale c that moves up to the
// largest key exponent seen so far (what is kept is multiplied by exp(c_old - c_new) when it
// does); the chunk's key features are stored on their own token's scale m_j (largest exponent of
// key j); and query i is evaluated on the scale P_i = max(c of the state it reads, m_j for the
// chunk's keys j <= i), the largest exponent among the keys it attends to: every weight is then
// at most 1 and the largest one is not below fp32's range, however far apart the exponents of
// different tokens are.  So A_ij enters as (f(q_i) . phi~(k_j)) exp(m_j - P_i), the carried state
// as exp(c_prev - P_i) S, and the state update as (exp(m_j - c) phi~(K))^T V: a second copy of the
// chunk's key features, Kc, is written already on the state's scale (where LDS has room for it;
// otherwise the factors go on the V operand).
//
// Feature order.  Features are stored in "operand order": stored feature q = 32 j + 8 g + 4 h + r
// is feature p = 32 j + 16 h + 4 g + r.  An MFMA result lane (g, r) of feature tiles 2j and
// 2j + 1 then writes 4 consecutive stored features, and the 8 k-slots a lane of group g gives a
// 16x16x32 operand over features are 8 consecutive stored features (one 16-byte LDS read).  The
// relabelling is the same in every tensor that carries a feature index (phi(K) tile, state, z,
// query features), so the products are unchanged; the state is converted back to feature order
// where it crosses the kernel's boundary.
//
// LDS (bf16 unless noted): Kf[C][M+16] phi(K_c) token-major (rows of M with pieces permuted by
// pswz where Kc exists); Kc[C][M+16] the same features on the state's scale (read by transpose
// reads, so padded); Vs[2][C][D] V of this chunk and the next; St[D][M] the state
// transposed, St[c][q] = S[q][c], pieces permuted by pswz; Zr[16][M+16] rows bf16(z) and
// bf16(z - bf16(z)); Ws[M][D+16] the projection.  Work per wave: one query tile, shared by
// waves w and 7 - w when C = 64 (they split the value columns), or its own when C = 128 (tiles
// w and 11 - w for the two waves of a SIMD, which balances the causal triangle); the same token
// tile (and half the features when two waves share it) for the next chunk's key projection; a
// block of the fp32 state accumulators (feature tiles NAW (w % 4).., column tiles NCW (w / 4)..;
// waves 0..3 also keep z).  C = 64 double-buffers V (the next chunk's V is stored while this one
// is read); C = 128 has LDS for one V tile only, stored with phi(K) between the barriers.
template <int D, int M, int C>
__global__ __launch_bounds__(512) void favor_causal(FavorCausalArgs a) {
  constexpr int NT = 512;
  constexpr int LDF = M + 16;      // padded rows: conflict-free 16-row operand and transpose reads
  constexpr int LDW = D + 16;
  constexpr int KA = D / 32;
  constexpr int MT = M / 16;       // feature tiles
  constexpr int MJ = M / 32;       // k-steps over features
  constexpr int NI = C / 16;       // token tiles per chunk
  constexpr int NQW = 8 / NI;      // waves per query tile
  constexpr int NVB = NQW;         // V buffers
  constexpr int NC = D / 16;       // value-column tiles
  constexpr int NAW = MT / 4;      // state feature tiles per wave
  constexpr int NCW = NC / 2;      // state column tiles per wave
  constexpr int OCT = NC / NQW;    // output column tiles per wave
  constexpr int HF = MT / NQW;     // key-projection feature tiles per wave
  constexpr int KJ = C / 32;       // k-steps over the tokens of a chunk
  constexpr int PPR = D / 8;
  constexpr int RPV = C * PPR / NT;
  constexpr int64_t REC = favor_rec(D, M);
  static_assert(NAW >= 1 && RPV >= 1 && OCT % 2 == 0 && (C == 64 || C == 128), "shape");
  // a second copy of the chunk's key features, on the state's scale, where LDS has room for it
  constexpr int kLdsBase = 2 * (C * LDF + NVB * C * D + D * LDF + 16 * LDF + M * LDW) +
                           4 * (8 + NQW * C + C);
  constexpr bool KCS = kLdsBase + 2 * C * LDF <= 160 * 1024;
  // chunks evaluated on the state's scale where the copy exists (64-token chunks: with 128 the
  // second path does not fit the registers)
  constexpr bool SAME = KCS && C == 64;

  __shared__ __attribute__((aligned(16))) uint16_t Kf[C * LDF];
  __shared__ __attribute__((aligned(16))) uint16_t Kc[KCS ? C * LDF : 8];  // phi(K_c), state's scale
  // Kf permuted (pswz) where only 16-row operand reads see it; with no Kc it is also the
  // transposed operand of the state update (ld_rows_operand), which wants the padded rows
  auto kfo = [](int t, int c) { return KCS ? pswz<M>(t, c) : t * LDF + c; };
  __shared__ __attribute__((aligned(16))) uint16_t Vs[NVB][C * D];
  __shared__ __attribute__((aligned(16))) uint16_t St[D * M];
  __shared__ __attribute__((aligned(16))) uint16_t Zr[16 * LDF];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[M * LDW];
  __shared__ float wmax[8];
  __shared__ __attribute__((aligned(16))) float tm[NQW][C];  // per-token maxima (per feature part)
  __shared__ __attribute__((aligned(16))) float mk[C];       // m_j of this chunk's keys

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.x / a.segs, seg = blockIdx.x % a.segs;
  const int64_t t0 = seg * a.seg_len;
  if (t0 >= a.n) return;
  const int64_t t1 = t0 + a.seg_len < a.n ? t0 + a.seg_len : a.n;
  const uint16_t* Q = reinterpret_cast<const uint16_t*>(a.q) + bh * a.n * D;
  const uint16_t* K = reinterpret_cast<const uint16_t*>(a.k) + bh * a.n * D;
  const uint16_t* V = reinterpret_cast<const uint16_t*>(a.v) + bh * a.n * D;
  uint16_t* O = reinterpret_cast<uint16_t*>(a.out) + bh * a.n * D;
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.w);

  // query tile, and token tile of the key projection; tile t belongs to wave wave_of(t) (and to
  // wave 7 - t as well when two waves share it)
  const int it = wave < 4 ? wave : (NQW == 2 ? 7 - wave : 11 - wave);
  auto wave_of = [](int t) { return t < 4 ? t : (NQW == 2 ? 7 - t : 11 - t); };
  const int part = (NQW == 2 && wave >= 4) ? 1 : 0;  // which half of a shared tile's work
  const int oc0 = part * OCT;                         // first output column tile
  const int hf0 = part * HF;                          // first key-projection feature tile
  const int sa0 = NAW * (wave & 3), sc0 = NCW * (wave >> 2);
  const bool zown = wave < 4;
  const float s = a.scale;
  const float kconst = 0.5f * logf((float)M);
  const float hs2 = 0.5f * s * s;
  const float sl2 = s * kLog2e;

  for (int e = tid; e < M * D / 8; e += NT) {
    const int f = e / (D / 8), c = (e % (D / 8)) * 8;
    st16(&Ws[f * LDW + c], ld16(W + f * D + c));
  }

  // ---- initial state: the leading segments' partial sums, brought to their largest log-scale
  f32x4 accS[NAW][NCW], accz[NAW];
#pragma unroll
  for (int i = 0; i < NAW; ++i) {
    accz[i] = zero4();
#pragma unroll
    for (int j = 0; j < NCW; ++j) accS[i][j] = zero4();
  }
  float c_cur = kNegInf;
  const int64_t nparts = seg * a.seg_parts;
  const float* parts = a.seg_state ? a.seg_state + bh * (a.segs - 1) * a.seg_parts * REC : nullptr;
  for (int64_t p = 0; p < nparts; ++p) c_cur = fmaxf(c_cur, parts[p * REC + (int64_t)M * D + M]);
  for (int64_t p = 0; p < nparts; ++p) {
    const float* rp = parts + p * REC;
    const float cp = rp[(int64_t)M * D + M];
    const float fac = cp == kNegInf ? 0.f : fexp(cp - c_cur);
#pragma unroll
    for (int i = 0; i < NAW; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pf = favor_p_of_q((sa0 + i) * 16 + 4 * g + r);
#pragma unroll
        for (int j = 0; j < NCW; ++j) accS[i][j][r] += fac * rp[(int64_t)pf * D + (sc0 + j) * 16 + l16];
        if (zown && l16 == 0) accz[i][r] += fac * rp[(int64_t)M * D + pf];
      }
    }
  }
  auto write_state = [&]() {
#pragma unroll
    for (int i = 0; i < NAW; ++i)
#pragma unroll
      for (int j = 0; j < NCW; ++j) {
        u32x2 w2;
        w2.x = pack_bf16(accS[i][j][0], accS[i][j][1]);
        w2.y = pack_bf16(accS[i][j][2], accS[i][j][3]);
        *reinterpret_cast<u32x2*>(&St[pswz<M>((sc0 + j) * 16 + l16, (sa0 + i) * 16 + g * 4)]) = w2;
      }
    if (zown && l16 == 0) {
#pragma unroll
      for (int i = 0; i < NAW; ++i) {
        u32x2 hi2, lo2;
        float hi[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) hi[r] = (float)(__bf16)accz[i][r];
        hi2.x = pack_bf16(hi[0], hi[1]);
        hi2.y = pack_bf16(hi[2], hi[3]);
        lo2.x = pack_bf16(accz[i][0] - hi[0], accz[i][1] - hi[1]);
        lo2.y = pack_bf16(accz[i][2] - hi[2], accz[i][3] - hi[3]);
        *reinterpret_cast<u32x2*>(&Zr[(sa0 + i) * 16 + g * 4]) = hi2;
        *reinterpret_cast<u32x2*>(&Zr[LDF + (sa0 + i) * 16 + g * 4]) = lo2;
      }
    }
  };
  for (int e = tid; e < 14 * LDF; e += NT) Zr[2 * LDF + e] = 0;  // rows 2..15 stay zero

  const uint32_t one2 = 0x3F803F80u;
  u32x4 ones;
  ones.x = ones.y = ones.z = ones.w = (l16 == 0) ? one2 : 0u;

  // ---- per-chunk row loads: the wave's key and query rows as MFMA operands (lane l16 = token,
  // k = 32 ks + 8 g), and 16-byte pieces of the V tile
  u32x4 kb[KA], qr[KA], vv[RPV];
  auto prow = [&](int p) { return tid / PPR + p * (NT / PPR); };
  const int pcol = (tid % PPR) * 8;
  auto load_kv = [&](int64_t c0) {
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) kb[ks] = ld16_clamp(K, c0 + it * 16 + l16, t1, D, ks * 32 + g * 8);
#pragma unroll
    for (int p = 0; p < RPV; ++p) vv[p] = ld16_clamp(V, c0 + prow(p), t1, D, pcol);
  };
  auto load_q = [&](int64_t c0) {
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) qr[ks] = ld16_clamp(Q, c0 + it * 16 + l16, t1, D, ks * 32 + g * 8);
  };
  auto store_v = [&](uint16_t* Vt, int64_t c0) {
#pragma unroll
    for (int p = 0; p < RPV; ++p) st16(&Vt[vofs<D>(prow(p), pcol)], keep_if(vv[p], c0 + prow(p) < t1));
  };
  // key projection of the loaded rows: u[ft][r] = exponent of feature 16 (hf0 + ft) + 4 g + r of
  // token l16 (-inf past the segment end); returns the wave's maximum
  f32x4 uk[HF];
  auto key_exponents = [&](int64_t c0) {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) ss = sumsq_bf16x8(kb[ks], ss);
    ss = sum_over_rows(ss);
    const bool ok = c0 + it * 16 + l16 < t1;
    const float off = ok ? hs2 * ss + kconst : __builtin_huge_valf();
    float mx = kNegInf;
#pragma unroll
    for (int ft = 0; ft < HF; ++ft) {
      uk[ft] = zero4();
#pragma unroll
      for (int ks = 0; ks < KA; ++ks)
        uk[ft] = mfma_bf16(ld16(&Ws[((hf0 + ft) * 16 + l16) * LDW + ks * 32 + g * 8]), kb[ks], uk[ft]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uk[ft][r] = s * uk[ft][r] - off;
        mx = fmaxf(mx, uk[ft][r]);
      }
    }
    // this half's maximum for token l16 (lanes l16, l16 + 16, ...), and the wave's maximum
    mx = max_over_groups(mx);
    if (g == 0) tm[part][it * 16 + l16] = mx;
    return wave_max(mx);
  };
  // phi(K) of the projected rows on their token's scale, into Kf (operand order), and the same
  // features on the scale c_state of the state they are added to, into Kc: exp(u - c) =
  // exp(u - m_j) exp(m_j - c), so that the state update takes V as it is; a token past the end
  // (all exponents -inf) gets zero features in both
  auto token_max = [&](int t) { return NQW == 2 ? fmaxf(tm[0][t], tm[NQW - 1][t]) : tm[0][t]; };
  // A chunk evaluated on its state's scale (same_scale) reads only Kc: Kf is not written, and
  // Kc is exp(u - c) directly.
  auto store_kf = [&](float c_state, bool same_scale) {
    const int t = it * 16 + l16;
    if constexpr (SAME) {
      if (same_scale) {
        const float c_l2 = c_state * kLog2e;
#pragma unroll
        for (int ft = 0; ft < HF; ++ft) {
          const int f = hf0 + ft;
          u32x2 c2;
          c2.x = pack_bf16(fexp_shift(uk[ft][0], kLog2e, c_l2), fexp_shift(uk[ft][1], kLog2e, c_l2));
          c2.y = pack_bf16(fexp_shift(uk[ft][2], kLog2e, c_l2), fexp_shift(uk[ft][3], kLog2e, c_l2));
          *reinterpret_cast<u32x2*>(&Kc[t * LDF + 32 * (f >> 1) + 8 * g + 4 * (f & 1)]) = c2;
        }
        return;
      }
    }
    const float mt = token_max(t);
    const float sh_l2 = mt == kNegInf ? 0.f : mt * kLog2e;
    const float et = (mt == kNegInf || c_state == kNegInf) ? 0.f : fexp(mt - c_state);
#pragma unroll
    for (int ft = 0; ft < HF; ++ft) {
      const int f = hf0 + ft;
      float w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = fexp_shift(uk[ft][r], kLog2e, sh_l2);
      u32x2 w2;
      w2.x = pack_bf16(w[0], w[1]);
      w2.y = pack_bf16(w[2], w[3]);
      const int col = 32 * (f >> 1) + 8 * g + 4 * (f & 1);
      *reinterpret_cast<u32x2*>(&Kf[kfo(t, col)]) = w2;
      if constexpr (KCS) {
        u32x2 c2;
        c2.x = pack_bf16(w[0] * et, w[1] * et);
        c2.y = pack_bf16(w[2] * et, w[3] * et);
        *reinterpret_cast<u32x2*>(&Kc[t * LDF + col]) = c2;
      }
    }
  };
  // m_j of the chunk's tokens (into mk, one wave per token tile) and P_i of this lane's query:
  // max(c_state, the maxima of the earlier token tiles (from the waves' maxima in wmax), the
  // prefix maximum within its own tile)
  auto chunk_maxima = [&](float c_state) {
    const int t = it * 16 + l16;
    float x = token_max(t);
    if (part == 0 && g == 0) mk[t] = x;
    x = prefix_max16(x);
    float base = c_state;
    for (int tp = 0; tp < it; ++tp)
      base = fmaxf(base, NQW == 2 ? fmaxf(wmax[tp], wmax[7 - tp]) : wmax[wave_of(tp)]);
    return fmaxf(base, x);
  };

  // ---- first chunk
  load_kv(t0);
  load_q(t0);
  __syncthreads();  // Ws ready
  {
    const float m0 = key_exponents(t0);
    if (lane == 0) wmax[wave] = m0;
  }
  store_v(Vs[0], t0);
  __syncthreads();
  float c_next = c_cur;
#pragma unroll
  for (int w = 0; w < 8; ++w) c_next = fmaxf(c_next, wmax[w]);
  float al = c_cur == kNegInf ? 0.f : fexp(c_cur - c_next);
  // whether the coming chunk is evaluated on its state's scale: its key maxima (token 0's is
  // the smallest P_i) within kSameScale of c_next
  bool same_next = SAME && __builtin_amdgcn_readfirstlane(
                               (int)(c_next - fmaxf(c_cur, token_max(0)) <= kSameScale));
  store_kf(c_next, same_next);
  // P_i of this lane's query in the coming chunk (and the chunk's key maxima mk), which a chunk
  // evaluated on its state's scale does not use
  float pq = same_next ? 0.f : chunk_maxima(c_cur);
  write_state();  // the initial state, on scale c_cur
  float c_prev = c_cur;  // scale of the state in St
  c_cur = c_next;        // scale of the state after this chunk
  bool same_cur = same_next;

  int buf = 0;
  for (int64_t c0 = t0; c0 < t1; c0 += C, buf ^= (NVB - 1)) {
    __syncthreads();  // Kf, Vs[buf], St, Zr of this chunk ready
    const uint16_t* Vc = Vs[buf];
    __builtin_amdgcn_sched_barrier(0);
    load_kv(c0 + C);
    __builtin_amdgcn_sched_barrier(0);

    // query features of this chunk's tile: U^T = W Q^T, f = exp(scale (U - max_f U))
    u32x4 fq[MJ];
    {
      f32x4 uq[MT];
      float mq = kNegInf;
#pragma unroll
      for (int ft = 0; ft < MT; ++ft) {
        uq[ft] = zero4();
#pragma unroll
        for (int ks = 0; ks < KA; ++ks)
          uq[ft] = mfma_bf16(ld16(&Ws[(ft * 16 + l16) * LDW + ks * 32 + g * 8]), qr[ks], uq[ft]);
#pragma unroll
        for (int r = 0; r < 4; ++r) mq = fmaxf(mq, uq[ft][r]);
      }
      mq = max_over_groups(mq);
      const float mq_l2 = mq * sl2;
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        fq[j].x = pack_bf16(fexp_shift(uq[2 * j][0], sl2, mq_l2), fexp_shift(uq[2 * j][1], sl2, mq_l2));
        fq[j].y = pack_bf16(fexp_shift(uq[2 * j][2], sl2, mq_l2), fexp_shift(uq[2 * j][3], sl2, mq_l2));
        fq[j].z = pack_bf16(fexp_shift(uq[2 * j + 1][0], sl2, mq_l2), fexp_shift(uq[2 * j + 1][1], sl2, mq_l2));
        fq[j].w = pack_bf16(fexp_shift(uq[2 * j + 1][2], sl2, mq_l2), fexp_shift(uq[2 * j + 1][3], sl2, mq_l2));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_q(c0 + C);
    __builtin_amdgcn_sched_barrier(0);

    // (i) state: rescale to this chunk's log-scale c (skipped when c did not move: al = 1 is the
    // usual case once the running maximum has settled), then S += phi(K_c)^T V_c and
    // z += phi(K_c)^T 1 with the key features on scale c (Kc)
    if (al != 1.f) {
#pragma unroll
      for (int i = 0; i < NAW; ++i) {
        accz[i] *= al;
#pragma unroll
        for (int j = 0; j < NCW; ++j) accS[i][j] *= al;
      }
    }
    if constexpr (KCS) {
      const u32x4 zones = zown ? ones : zero_u4();
#pragma unroll
      for (int ks = 0; ks < KJ; ++ks) {
        u32x4 bv[NCW];
#pragma unroll
        for (int j = 0; j < NCW; ++j) bv[j] = ld_v_rows<D>(Vc, ks * 32, (sc0 + j) * 16, l16, g);
#pragma unroll
        for (int i = 0; i < NAW; ++i) {
          const u32x4 ak = ld_rows_operand(Kc, LDF, ks * 32, (sa0 + i) * 16, l16, g);
          accz[i] = mfma_bf16(ak, zones, accz[i]);
#pragma unroll
          for (int j = 0; j < NCW; ++j) accS[i][j] = mfma_bf16(ak, bv[j], accS[i][j]);
        }
      }
    } else {
      // no room for the second copy: the factors e_j = exp(m_j - c) go on the V operand (and on
      // the ones column of z) instead
#pragma unroll
      for (int ks = 0; ks < KJ; ++ks) {
        const f32x4 m_lo = *reinterpret_cast<const f32x4*>(&mk[ks * 32 + 4 * g]);
        const f32x4 m_hi = *reinterpret_cast<const f32x4*>(&mk[ks * 32 + 16 + 4 * g]);
        float e8[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e8[r] = fexp(m_lo[r] - c_cur);
          e8[4 + r] = fexp(m_hi[r] - c_cur);
        }
        u32x4 bz;  // column 0: the factors; other columns zero
        bz.x = pack_bf16(e8[0], e8[1]);
        bz.y = pack_bf16(e8[2], e8[3]);
        bz.z = pack_bf16(e8[4], e8[5]);
        bz.w = pack_bf16(e8[6], e8[7]);
        bz = keep_if(bz, zown && l16 == 0);
        u32x4 bv[NCW];
#pragma unroll
        for (int j = 0; j < NCW; ++j) {
          const u32x4 raw = ld_v_rows<D>(Vc, ks * 32, (sc0 + j) * 16, l16, g);
          bv[j].x = pack_bf16(bf_lo(raw.x) * e8[0], bf_hi(raw.x) * e8[1]);
          bv[j].y = pack_bf16(bf_lo(raw.y) * e8[2], bf_hi(raw.y) * e8[3]);
          bv[j].z = pack_bf16(bf_lo(raw.z) * e8[4], bf_hi(raw.z) * e8[5]);
          bv[j].w = pack_bf16(bf_lo(raw.w) * e8[6], bf_hi(raw.w) * e8[7]);
        }
#pragma unroll
        for (int i = 0; i < NAW; ++i) {
          const u32x4 ak = ld_rows_operand(Kf, LDF, ks * 32, (sa0 + i) * 16, l16, g);
          accz[i] = mfma_bf16(ak, bz, accz[i]);
#pragma unroll
          for (int j = 0; j < NCW; ++j) accS[i][j] = mfma_bf16(ak, bv[j], accS[i][j]);
        }
      }
    }

    // (ii) earlier chunks: S^T f and [z_hi; z_lo] f on the previous scale, then rescaled
    f32x4 acco[OCT];
    f32x4 accd = zero4();
#pragma unroll
    for (int ct = 0; ct < OCT; ++ct) acco[ct] = zero4();
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
#pragma unroll
      for (int ct = 0; ct < OCT; ++ct)
        acco[ct] = mfma_bf16(ld16(&St[pswz<M>((oc0 + ct) * 16 + l16, 32 * j + 8 * g)]), fq[j], acco[ct]);
      accd = mfma_bf16(ld16(&Zr[l16 * LDF + 32 * j + 8 * g]), fq[j], accd);
    }
    // A chunk whose key maxima lie within kSameScale of its state's scale evaluates every query
    // on that scale c_cur instead of its own P_i (every weight still at most 1, the smallest
    // shrunk by at most e^-kSameScale, far inside the bf16 / fp32 range): the key features
    // already written on c_cur (Kc) are then the masked product's operand as they are, and the
    // carried state takes one factor for all queries.  Other chunks use P_i.
    const bool same = same_cur;
    const float pe = same ? c_cur : pq;  // the scale of this lane's query in this chunk
    const float pq_l2 = pe * kLog2e;
    {
      const float sc = fexp(c_prev - pe);
      if (sc != 1.f) {
#pragma unroll
        for (int ct = 0; ct < OCT; ++ct) acco[ct] *= sc;
        accd *= sc;
      }
    }

    // (iii) this chunk: A^T = phi(K_c) f^T masked to key <= query, then V^T A^T and ones A^T
    auto a_tiles = [&](int m, f32x4& a0, f32x4& a1, auto samec) {
      a0 = zero4();
      a1 = zero4();
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        if constexpr (decltype(samec)::value) {
          a0 = mfma_bf16(ld16(&Kc[(2 * m * 16 + l16) * LDF + 32 * j + 8 * g]), fq[j], a0);
          a1 = mfma_bf16(ld16(&Kc[((2 * m + 1) * 16 + l16) * LDF + 32 * j + 8 * g]), fq[j], a1);
        } else {
          a0 = mfma_bf16(ld16(&Kf[kfo(2 * m * 16 + l16, 32 * j + 8 * g)]), fq[j], a0);
          a1 = mfma_bf16(ld16(&Kf[kfo((2 * m + 1) * 16 + l16, 32 * j + 8 * g)]), fq[j], a1);
        }
      }
    };
    auto pack_a = [&](int m, f32x4 a0, f32x4 a1, auto samec, auto maskc) {
      if constexpr (!decltype(samec)::value) {
        const f32x4 m0 = *reinterpret_cast<const f32x4*>(&mk[32 * m + 4 * g]);
        const f32x4 m1 = *reinterpret_cast<const f32x4*>(&mk[32 * m + 16 + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          a0[r] *= fexp_shift(m0[r], kLog2e, pq_l2);
          a1[r] *= fexp_shift(m1[r], kLog2e, pq_l2);
        }
      }
      if constexpr (decltype(maskc)::value) {  // the last step holds the diagonal tile
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (2 * m == it && g * 4 + r > l16) a0[r] = 0.f;
          if (2 * m + 1 > it || (2 * m + 1 == it && g * 4 + r > l16)) a1[r] = 0.f;
        }
      }
      u32x4 af;
      af.x = pack_bf16(a0[0], a0[1]);
      af.y = pack_bf16(a0[2], a0[3]);
      af.z = pack_bf16(a1[0], a1[1]);
      af.w = pack_bf16(a1[2], a1[3]);
      return af;
    };
    auto av_step = [&](int m, u32x4 af) {
#pragma unroll
      for (int ct = 0; ct < OCT; ++ct) acco[ct] = mfma_bf16(ld_v_rows<D>(Vc, m * 32, (oc0 + ct) * 16, l16, g), af, acco[ct]);
      accd = mfma_bf16(ones, af, accd);
    };
    // step m covers key tiles 2m and 2m + 1; the A products of step m + 1 are issued before the
    // V products of step m so that the two overlap
    auto intra = [&](auto samec) {
      const int mlast = it >> 1;
      f32x4 a0, a1;
      a_tiles(0, a0, a1, samec);
#pragma unroll
      for (int m = 0; m < NI / 2 - 1; ++m) {
        if (m < mlast) {
          const u32x4 af = pack_a(m, a0, a1, samec, BoolC<false>{});  // below the diagonal
          a_tiles(m + 1, a0, a1, samec);
          av_step(m, af);
        }
      }
      av_step(mlast, pack_a(mlast, a0, a1, samec, BoolC<true>{}));
    };
    if constexpr (SAME) {
      if (same)
        intra(BoolC<true>{});
      else
        intra(BoolC<false>{});
    } else {
      intra(BoolC<false>{});
    }

    const float den = from_row0(accd[0] + accd[1]);
    const float inv = 1.0f / den;
    const int64_t row = c0 + it * 16 + l16;
#pragma unroll
    for (int ct = 0; ct < OCT; ct += 2) {
      const uint32_t ax = pack_bf16(acco[ct][0] * inv, acco[ct][1] * inv);
      const uint32_t ay = pack_bf16(acco[ct][2] * inv, acco[ct][3] * inv);
      const uint32_t bx = pack_bf16(acco[ct + 1][0] * inv, acco[ct + 1][1] * inv);
      const uint32_t by = pack_bf16(acco[ct + 1][2] * inv, acco[ct + 1][3] * inv);
      const auto sx = __builtin_amdgcn_permlane16_swap(ax, bx, false, false);
      const auto sy = __builtin_amdgcn_permlane16_swap(ay, by, false, false);
      u32x4 o;
      o.x = sx[0];
      o.y = sy[0];
      o.z = sx[1];
      o.w = sy[1];
      if (row < t1) st16(O + row * D + (oc0 + ct + (g & 1)) * 16 + 8 * (g >> 1), o);
    }

    // next chunk: key exponents and their maximum, V to the idle buffer (if there is one)
    {
      const float mn = key_exponents(c0 + C);
      if (lane == 0) wmax[wave] = mn;
    }
    if (NVB == 2) store_v(Vs[buf ^ 1], c0 + C);
    __syncthreads();  // every wave is done with Kf, Vs, St, Zr of this chunk; the maxima are in
    c_next = c_cur;
#pragma unroll
    for (int w = 0; w < 8; ++w) c_next = fmaxf(c_next, wmax[w]);
    al = fexp(c_cur - c_next);
    if (NVB == 1) store_v(Vs[0], c0 + C);
    same_next = SAME && __builtin_amdgcn_readfirstlane(
                            (int)(c_next - fmaxf(c_cur, token_max(0)) <= kSameScale));
    store_kf(c_next, same_next);
    pq = same_next ? 0.f : chunk_maxima(c_cur);
    write_state();  // the state after this chunk, on scale c_cur
    c_prev = c_cur;
    c_cur = c_next;
    same_cur = same_next;
  }

  // the state after the last token (scale c_cur), in feature order, from the last segment
  if (a.sn && seg == (a.n - 1) / a.seg_len) {
    float* sn = a.sn + bh * M * D;
#pragma unroll
    for (int i = 0; i < NAW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pf = favor_p_of_q((sa0 + i) * 16 + 4 * g + r);
#pragma unroll
        for (int j = 0; j < NCW; ++j) sn[(int64_t)pf * D + (sc0 + j) * 16 + l16] = accS[i][j][r];
        if (zown && l16 == 0) a.zn[bh * M + pf] = accz[i][r];
      }
    if (tid == 0) a.cn[bh] = c_cur;
  }
}

template <int D, int M>
__global__ __launch_bounds__(256) void favor_empty_state(FavorCausalArgs a) {
  const int64_t h = blockIdx.x;
  for (int e = threadIdx.x; e < M * D; e += 256) a.sn[h * M * D + e] = 0.f;
  for (int e = threadIdx.x; e < M; e += 256) a.zn[h * M + e] = 0.f;
  if (threadIdx.x == 0) a.cn[h] = kNegInf;
}

// ================================================================ launchers
template <class F>
static hipError_t favor_dispatch(int d, int m, F&& f) {
  if (d == 64 && m == 64) f(std::integral_constant<int, 64>{}, std::integral_constant<int, 64>{});
  else if (d == 64 && m == 128) f(std::integral_constant<int, 64>{}, std::integral_constant<int, 128>{});
  else if (d == 64 && m == 256) f(std::integral_constant<int, 64>{}, std::integral_constant<int, 256>{});
  else if (d == 128 && m == 64) f(std::integral_constant<int, 128>{}, std::integral_constant<int, 64>{});
  else if (d == 128 && m == 128) f(std::integral_constant<int, 128>{}, std::integral_constant<int, 128>{});
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_favor_kv_state(const FavorStateArgs& a, int d, int m, hipStream_t s) {
  return favor_dispatch(d, m, [&](auto Dc, auto Mc) {
    hipLaunchKernelGGL((favor_kv_state<decltype(Dc)::value, decltype(Mc)::value>),
                       dim3((unsigned)(a.groups * a.slices)), dim3(FAVOR_NW(decltype(Dc)::value, decltype(Mc)::value) * 64), 0, s, a);
  });
}

hipError_t launch_favor_reduce(const FavorReduceArgs& a, int d, int m, hipStream_t s) {
  return favor_dispatch(d, m, [&](auto Dc, auto Mc) {
    hipLaunchKernelGGL((favor_reduce<decltype(Dc)::value, decltype(Mc)::value>),
                       dim3((unsigned)(a.groups * 8)), dim3(256), 0, s, a);
  });
}

hipError_t launch_favor_out(const FavorOutArgs& a, int d, int m, hipStream_t s) {
  const int64_t blocks = a.bh * ((a.n + kFavorQueries - 1) / kFavorQueries);
  return favor_dispatch(d, m, [&](auto Dc, auto Mc) {
    hipLaunchKernelGGL((favor_out<decltype(Dc)::value, decltype(Mc)::value>), dim3((unsigned)blocks),
                       dim3(512), 0, s, a);
  });
}

hipError_t launch_favor_decode(const FavorDecodeArgs& a, int d, int m, hipStream_t s) {
  return favor_dispatch(d, m, [&](auto Dc, auto Mc) {
    hipLaunchKernelGGL((favor_decode<decltype(Dc)::value, decltype(Mc)::value>), dim3((unsigned)a.bh),
                       dim3(256), 0, s, a);
  });
}

}  // namespace la

namespace la {

hipError_t launch_favor_causal(const FavorCausalArgs& a, int d, int m, int chunk, hipStream_t s) {
  return favor_dispatch(d, m, [&](auto Dc, auto Mc) {
    constexpr int D = decltype(Dc)::value, M = decltype(Mc)::value;
    if constexpr (favor_chunk_ok(D, M, 128)) {
      if (chunk == 128) {
        hipLaunchKernelGGL((favor_causal<D, M, 128>), dim3((unsigned)(a.bh * a.segs)), dim3(512), 0, s, a);
        return;
      }
    }
    hipLaunchKernelGGL((favor_causal<D, M, 64>), dim3((unsigned)(a.bh * a.segs)), dim3(512), 0, s, a);
  });
}

hipError_t launch_favor_empty_state(const FavorCausalArgs& a, int d, int m, hipStream_t s) {
  return favor_dispatch(d, m, [&](auto Dc, auto Mc) {
    hipLaunchKernelGGL((favor_empty_state<decltype(Dc)::value, decltype(Mc)::value>), dim3((unsigned)a.bh),
                       dim3(256), 0, s, a);
  });
}

}  // namespace la
