// la_causal.hip -- causal (j <= i) linear attention, chunked, on gfx950.
//
// Math ("Efficient Transformers: Linear Attention and Flash Attention", section "The recurrent
// view: attention as an RNN"): out_i = phi(q_i)^T S_i / phi(q_i)^T z_i with the prefix sums
// S_i = sum_{j<=i} phi(k_j) v_j^T and z_i = sum_{j<=i} phi(k_j).  Split the keys of a query in
// chunk [c0, c0+C) at c0 (associativity, section "Linear attention: reordering the matmuls"):
//   j <  c0  : the running state (S, z) carried from earlier chunks,
//   c0 <= j <= i : the masked pairwise weights A_ij = phi(q_i).phi(k_j) inside the chunk,
// so  num_i = sum_j A_ij v_j + phi(q_i)^T S,  den_i = sum_j A_ij + phi(q_i)^T z,  and after the
// chunk S += phi(K_c)^T V_c, z += phi(K_c)^T 1.
//
// Work split.  One workgroup walks one segment of one head chunk by chunk; a head is cut into
// `segs` segments so that short batches still fill the GPU.  The state entering segment s is
// the state before the sequence (zero, or a caller's (S0, z0)) plus the leading segments'
// state sums, computed beforehand by the stage-1 kernel of la_noncausal.hip (any partition of
// the keys gives the same sums).  The workgroup of the last segment can write the state after
// the last token: the recurrence's state, handed on to a later call or to the decode step.
#include "la_common.h"
#include "la_kernels.h"

namespace la {

// Initial (S, z) of a segment: the sum over the leading segments' parts, in order
// (segment s', part p) -> index (s' * seg_parts + p).
__device__ __forceinline__ const float* seg_state_ptr(const CausalArgs& a, int64_t bh, int64_t sp,
                                                      int D) {
  return a.seg_state + (bh * (a.segs - 1) * a.seg_parts + sp) * (int64_t)(D * D + D);
}

// bf16 kernel, D = head dim, C = chunk.  512 threads = 8 waves; waves w and w+4 share SIMD w%4.
//
// LDS (bf16 unless noted), all row-major:
//   Kn[C][D]      phi(K) of the chunk, token-major, row stride D + 16;
//   Vn[2][C][D]   V of this chunk and of the next one (stored while this one is in use),
//                 token-major, rows of D elements with the 16-byte pieces of row r permuted;
//   St[D][D]      the running state transposed, St[c][a] = S[a][c], rounded to bf16, 16-byte
//                 pieces permuted by the row (pswz);
//   Zr[16][D]     a normaliser tile: row 0 = bf16(z), row 1 = bf16(z - row 0), rows 2..15 zero;
//   zf[D]         fp32 z at the segment start.
// Operands whose reduction index is the token (phi(K)^T and V in the state update, V^T in the
// masked product) come straight from the token-major tiles through LDS transpose reads, so
// nothing is transposed in registers and each tile is stored once.
//
// Pipeline: the K and V tiles and the query rows of chunk c + 1 are loaded into registers
// (non-temporal loads: each is read once; measured faster than loads that allocate in the caches)
// while chunk c is computed (at points spread over the chunk, so that the memory queue does
// not stall the issuing waves); V(c + 1) goes to the idle V buffer before the chunk's second
// barrier, phi(K(c + 1)) to Kn after it, together with the new state and the outputs'
// global stores.
//
// Work per wave:
//   * one query tile of 16 rows (C = 128: tile w for w < 4, 11 - w otherwise, so the two waves
//     of a SIMD hold tiles s and 7 - s and share the masked triangle evenly; C = 64: four
//     tiles for eight waves, tile w or 7 - w, each wave taking half of the value columns);
//   * a 2-D block of the fp32 state accumulators: feature tiles NAW*(w%4).., value-column
//     tiles NCW*(w/4)..; waves 0..3 also keep z for their feature tiles.
// Outputs are computed transposed, out^T[c][i] (c = MFMA row, query = MFMA column), so that
//   * phi(Q) needs no LDS: a lane's 16-byte load of its query row is its operand;
//   * the masked tile is computed as A^T[j][i] = phi(K) phi(Q)^T; in the MFMA result a lane
//     holds j = 16*jt + 4g + r for its query, so two j-tiles give 8 j values per lane, which
//     is the operand layout of the next product with the k index permuted accordingly;
//     V is read with the same permutation, and A never goes through LDS;
//   * the normaliser rides along as one extra 16-row output tile: z (hi, lo) rows against
//     phi(Q) and a row of ones against A give phi(q).z + sum_j A_ij in rows 0 and 1.
template <int D, int C, class TB>
__global__ __launch_bounds__(512) void causal_bf16(CausalArgs a, TB tb) {
  constexpr int NT = 512;
  constexpr int LDK = D + 16;       // row stride of 8 mod 64 dwords: conflict-free 16-row reads
  constexpr int NI = C / 16;         // query (and key) tiles per chunk
  constexpr int NC = D / 16;         // value-column tiles
  constexpr int NA = D / 16;         // feature tiles
  constexpr int NAW = NA / 4;        // state feature tiles per wave
  constexpr int NCW = NC / 2;        // state value-column tiles per wave
  constexpr int OCT = NI == 8 ? NC : NC / 2;   // output column tiles per wave
  constexpr int KA = D / 32;         // k-steps over features
  constexpr int KJ = C / 32;         // k-steps over tokens
  constexpr int PPR = D / 8;          // 16-byte pieces per row
  constexpr int RPK = C * PPR / NT;   // K pieces per thread
  static_assert(NI == 8 || NI == 4, "chunk");
  static_assert(RPK >= 1, "tile split");

  __shared__ __attribute__((aligned(16))) uint16_t Kn[C * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Vn[2 * C * D];
  __shared__ __attribute__((aligned(16))) uint16_t St[D * D];
  __shared__ __attribute__((aligned(16))) uint16_t Zr[16 * LDK];
  __shared__ float zf[D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.x / a.segs, seg = blockIdx.x % a.segs;
  const HeadSpan sp = head_span(tb, a.n, bh);
  const int64_t t0 = seg * a.seg_len;
  if (t0 >= sp.n) return;  // a segment past a shorter sequence's end (variable lengths)
  const int64_t t1 = t0 + a.seg_len < sp.n ? t0 + a.seg_len : sp.n;
  const uint16_t* Q = reinterpret_cast<const uint16_t*>(a.q) + sp.row0 * D;
  const uint16_t* K = reinterpret_cast<const uint16_t*>(a.k) + sp.row0 * D;
  const uint16_t* V = reinterpret_cast<const uint16_t*>(a.v) + sp.row0 * D;
  uint16_t* O = reinterpret_cast<uint16_t*>(a.out) + sp.row0 * D;

  const int it = wave < 4 ? wave : (NI == 8 ? 11 - wave : 7 - wave);   // this wave's query tile
  const int oc0 = (NI == 8 || wave < 4) ? 0 : NC / 2;                 // its first output column tile
  const int sa0 = NAW * (wave & 3), sc0 = NCW * (wave >> 2);           // its state block
  const bool zown = wave < 4;                                          // keeps z of tiles sa0..

  // ---- initial state: sum of the leading segments' sums
  f32x4 accS[NAW][NCW];
#pragma unroll
  for (int i = 0; i < NAW; ++i)
#pragma unroll
    for (int j = 0; j < NCW; ++j) accS[i][j] = zero4();
  float zinit = 0.f;
  if (a.s0) {  // the state before the sequence
    const float* s0 = a.s0 + bh * D * D;
#pragma unroll
    for (int i = 0; i < NAW; ++i)
#pragma unroll
      for (int j = 0; j < NCW; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) accS[i][j][r] = s0[((sa0 + i) * 16 + g * 4 + r) * D + (sc0 + j) * 16 + l16];
    if (tid < D) zinit = a.z0[bh * D + tid];
  }
  // per leading segment: add its parts in order, then add the segment (the same grouping as
  // la_state_sums followed by la_causal_segments, so both paths round identically)
  for (int64_t s = 0; s < seg; ++s) {
    f32x4 part[NAW][NCW];
    float zpart = 0.f;
#pragma unroll
    for (int i = 0; i < NAW; ++i)
#pragma unroll
      for (int j = 0; j < NCW; ++j) part[i][j] = zero4();
    for (int64_t p = 0; p < a.seg_parts; ++p) {
      const float* st = seg_state_ptr(a, bh, s * a.seg_parts + p, D);
#pragma unroll
      for (int i = 0; i < NAW; ++i)
#pragma unroll
        for (int j = 0; j < NCW; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            part[i][j][r] += st[((sa0 + i) * 16 + g * 4 + r) * D + (sc0 + j) * 16 + l16];
      if (tid < D) zpart += st[D * D + tid];
    }
#pragma unroll
    for (int i = 0; i < NAW; ++i)
#pragma unroll
      for (int j = 0; j < NCW; ++j) accS[i][j] += part[i][j];
    zinit += zpart;
  }
  if (tid < D) zf[tid] = zinit;
  auto write_state_bf16 = [&]() {
#pragma unroll
    for (int i = 0; i < NAW; ++i)
#pragma unroll
      for (int j = 0; j < NCW; ++j) {
        u32x2 w2;
        w2.x = pack_bf16(accS[i][j][0], accS[i][j][1]);
        w2.y = pack_bf16(accS[i][j][2], accS[i][j][3]);
        *reinterpret_cast<u32x2*>(&St[pswz<D>((sc0 + j) * 16 + l16, (sa0 + i) * 16 + g * 4)]) = w2;
      }
  };
  write_state_bf16();
  __syncthreads();
  const uint32_t one2 = 0x3F803F80u;  // two bf16 ones
  u32x4 ones;                          // B operand with a column of ones (column 0)
  ones.x = ones.y = ones.z = ones.w = (l16 == 0) ? one2 : 0u;
  // z of this wave's feature tiles, kept as an MFMA accumulator: phi(K)^T [1 0 ... 0] puts the
  // key sums in column 0, i.e. in lanes with l16 == 0, rows 4g + r
  f32x4 accz[NAW];
  const u32x4 zones = zown ? ones : zero_u4();
#pragma unroll
  for (int i = 0; i < NAW; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) accz[i][r] = (zown && l16 == 0) ? zf[(sa0 + i) * 16 + g * 4 + r] : 0.f;
  for (int e = tid; e < 16 * D; e += NT) {
    const int row = e / D, c = e % D;
    uint16_t val = 0;
    if (row < 2) {
      const float z = zf[c];
      const __bf16 hi = (__bf16)z;
      val = row == 0 ? __builtin_bit_cast(uint16_t, hi) : __builtin_bit_cast(uint16_t, (__bf16)(z - (float)hi));
    }
    Zr[row * LDK + c] = val;
  }

  // ---- K and V tiles: piece tid + 512 p of each (16 consecutive lanes cover one 256-byte row
  // when D = 128)
  u32x4 kv[RPK], vv[RPK];
  u32x4 qr[KA];  // this wave's query rows (raw)
  auto prow = [&](int p) { return tid / PPR + p * (NT / PPR); };
  const int pcol = (tid % PPR) * 8;
  auto load_k = [&](int64_t c0) {
#pragma unroll
    for (int p = 0; p < RPK; ++p) kv[p] = ld16_clamp_nt(K, c0 + prow(p), t1, D, pcol);
  };
  auto load_v = [&](int64_t c0) {
#pragma unroll
    for (int p = 0; p < RPK; ++p) vv[p] = ld16_clamp_nt(V, c0 + prow(p), t1, D, pcol);
  };
  // feature map on K; rows past the segment end become zero in both tiles
  auto prep_kv = [&](int64_t c0) {
#pragma unroll
    for (int p = 0; p < RPK; ++p) {
      const bool ok = c0 + prow(p) < t1;
      kv[p] = keep_if(phi_bf16x8(kv[p]), ok);
      vv[p] = keep_if(vv[p], ok);
    }
  };
  auto store_k = [&]() {
#pragma unroll
    for (int p = 0; p < RPK; ++p) st16(&Kn[prow(p) * LDK + pcol], kv[p]);
  };
  auto load_q = [&](int64_t c0) {
    const int64_t row = c0 + it * 16 + l16;
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) qr[ks] = ld16_clamp_nt(Q, row, t1, D, ks * 32 + g * 8);  // rows >= t1 are never stored
  };

  // ---- V tiles.  Piece permutation: the 8 rows that a half-wave transpose read touches fall
  // on distinct bank groups (rows of 256 bytes: one row per 64 banks; of 128 bytes: two).
  constexpr int VRL = 128 / D;
  auto vofs = [&](int r, int c) { return r * D + ((((c >> 3) ^ (2 * ((r / VRL) % (D / 16))))) << 3) + (c & 7); };
  // 16x16x32 operand with k over the rows of a V tile (the layout of ld_rows_operand); rows
  // r and r + 16 share their permutation
  auto ld_v_operand = [&](const uint16_t* Vt, int row0, int col0) {
    const uint16_t* p0 = Vt + vofs(row0 + 4 * g + (l16 >> 2), col0 + 4 * (l16 & 3));
    const u32x2 lo = ld_tr16(p0), hi = ld_tr16(p0 + 16 * D);
    u32x4 r;
    r.x = lo.x;
    r.y = lo.y;
    r.z = hi.x;
    r.w = hi.y;
    return r;
  };
  auto store_v = [&](uint16_t* Vt) {
#pragma unroll
    for (int p = 0; p < RPK; ++p) st16(&Vt[vofs(prow(p), pcol)], vv[p]);
  };

  if (t0 < t1) {
    load_k(t0);
    load_v(t0);
    load_q(t0);
    prep_kv(t0);
    store_k();
    store_v(Vn);
  }
  int buf = 0;
  for (int64_t c0 = t0; c0 < t1; c0 += C, buf ^= 1) {
    __syncthreads();  // tiles of this chunk, St, Zr ready
    const uint16_t* Vc = Vn + buf * (C * D);
    // Loads for the next chunk go out in three groups (K here, V after the state update, the
    // query rows after the inter-chunk product), pinned in place by scheduling barriers: one
    // burst of all of them would fill the memory queue and stall the issuing waves.  Every
    // thread loads at the same points, unconditionally (rows past the end are clamped):
    // loads under a condition would join the loop-carried registers through copies that wait
    // for the data on the spot.
    __builtin_amdgcn_sched_barrier(0);
    load_k(c0 + C);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 qf[KA];
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) qf[ks] = phi_bf16x8(qr[ks]);

    // ---- (iv) state update in registers: S[own block] += phi(K_c)^T V_c ; z
#pragma unroll
    for (int ks = 0; ks < KJ; ++ks) {
      u32x4 bv[NCW];
#pragma unroll
      for (int j = 0; j < NCW; ++j) bv[j] = ld_v_operand(Vc, ks * 32, (sc0 + j) * 16);
#pragma unroll
      for (int i = 0; i < NAW; ++i) {
        const u32x4 ak = ld_rows_operand(Kn, LDK, ks * 32, (sa0 + i) * 16, l16, g);
        accz[i] = mfma_bf16(ak, zones, accz[i]);  // no branch: zones is zero where z is not kept
#pragma unroll
        for (int j = 0; j < NCW; ++j) accS[i][j] = mfma_bf16(ak, bv[j], accS[i][j]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_v(c0 + C);
    __builtin_amdgcn_sched_barrier(0);

    // ---- this wave's query tile: inter-chunk part, then the masked intra-chunk part one
    // 32-key step at a time (A^T for key tiles 2m and 2m+1 goes straight into the V product)
    f32x4 acco[OCT];
    f32x4 accd = zero4();
#pragma unroll
    for (int ct = 0; ct < OCT; ++ct) acco[ct] = zero4();
    // inter-chunk: S^T phi(Q)^T and [z_hi; z_lo] phi(Q)^T
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) {
#pragma unroll
      for (int ct = 0; ct < OCT; ++ct)
        acco[ct] = mfma_bf16(ld16(&St[pswz<D>((oc0 + ct) * 16 + l16, ks * 32 + g * 8)]), qf[ks], acco[ct]);
      accd = mfma_bf16(ld16(&Zr[l16 * LDK + ks * 32 + g * 8]), qf[ks], accd);
    }
    __builtin_amdgcn_sched_barrier(0);
    load_q(c0 + C);
    __builtin_amdgcn_sched_barrier(0);
    // intra-chunk: A^T = phi(K) phi(Q)^T masked to key <= query, then V^T A^T and ones A^T.
    // Step m covers key tiles 2m and 2m+1; the A^T products of step m+1 are issued before the
    // V products of step m so that the two overlap.  A key tile past the query tile is zeroed.
    auto a_tiles = [&](int m, f32x4& a0, f32x4& a1) {
      a0 = zero4();
      a1 = zero4();
#pragma unroll
      for (int ks = 0; ks < KA; ++ks) {
        a0 = mfma_bf16(ld16(&Kn[(2 * m * 16 + l16) * LDK + ks * 32 + g * 8]), qf[ks], a0);
        a1 = mfma_bf16(ld16(&Kn[((2 * m + 1) * 16 + l16) * LDK + ks * 32 + g * 8]), qf[ks], a1);
      }
    };
    auto pack_a = [&](int m, f32x4 a0, f32x4 a1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (2 * m == it && g * 4 + r > l16) a0[r] = 0.f;
        if (2 * m + 1 > it || (2 * m + 1 == it && g * 4 + r > l16)) a1[r] = 0.f;
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
      for (int ct = 0; ct < OCT; ++ct)
        acco[ct] = mfma_bf16(ld_v_operand(Vc, m * 32, (oc0 + ct) * 16), af, acco[ct]);
      accd = mfma_bf16(ones, af, accd);
    };
    const int mlast = it >> 1;
    f32x4 a0, a1;
    a_tiles(0, a0, a1);
#pragma unroll
    for (int m = 0; m < NI / 2 - 1; ++m) {
      if (m < mlast) {
        const u32x4 af = pack_a(m, a0, a1);
        a_tiles(m + 1, a0, a1);
        av_step(m, af);
      }
    }
    av_step(mlast, pack_a(mlast, a0, a1));

    const float den = __shfl(accd[0] + accd[1], l16);
    const float inv = 1.0f / den;
    // Outputs: a lane holds 4 columns of each column tile.  For a pair of tiles (ct, ct + 1)
    // lane rows g and g ^ 1 swap halves (v_permlane16_swap: odd rows of the first operand with
    // even rows of the second), so that a lane of row g holds 8 consecutive columns of tile
    // ct + (g & 1), starting at 8 (g / 2): one 16-byte store.
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
    // next chunk's tiles (past the last chunk these are zero tiles that nothing reads); its V
    // goes to the idle buffer at once
    prep_kv(c0 + C);
    store_v(Vn + (buf ^ 1) * (C * D));
    __syncthreads();  // every wave is done reading this chunk's Kn, St and Zr

    // ---- the next chunk's phi(K), the new state
    store_k();
    write_state_bf16();
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
        *reinterpret_cast<u32x2*>(&Zr[LDK + (sa0 + i) * 16 + g * 4]) = lo2;
      }
    }
  }

  // the state after the last token, from the last segment's workgroup
  if (a.sn && seg == (sp.n - 1) / a.seg_len) {
    float* sn = a.sn + bh * D * D;
#pragma unroll
    for (int i = 0; i < NAW; ++i)
#pragma unroll
      for (int j = 0; j < NCW; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) sn[((sa0 + i) * 16 + g * 4 + r) * D + (sc0 + j) * 16 + l16] = accS[i][j][r];
    if (zown && l16 == 0) {
#pragma unroll
      for (int i = 0; i < NAW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) a.zn[bh * D + (sa0 + i) * 16 + g * 4 + r] = accz[i][r];
    }
  }
}

// waves per workgroup of the fp32 kernel: eight at d = 128, whose LDS admits one workgroup per
// compute unit (four waves would leave one wave per SIMD), four otherwise
constexpr int f32_waves(int d) { return d == 128 ? 8 : 4; }

// fp32 kernel (no bf16 rounding anywhere).  The fp32 MFMA takes one k value per lane; a lane
// holds 16-byte pieces of rows, features 16m + 4g .. 16m + 4g + 3, and k-step (m, e) pairs
// feature 16m + 4g + e on both operands.  With four waves, each wave owns query tiles (tiles w
// and NI - 1 - w when a chunk has 8, tile w when it has 4) and produces all output columns of
// them: the masked tile A^T = phi(K) phi(Q)^T of each (key tile, query tile) pair is computed
// once, by its owner, and fed back as an operand with permuted k, as in the bf16 kernel.  With
// eight waves (d = 128) waves w and 7 - w share tile w and produce half the columns each, both
// computing its masked tiles.  The inter-chunk product reads S^T from LDS; the state
// accumulators are split by value columns (wave w owns column tiles w, w + NW, ...) and written
// to S^T after each chunk's update.  The next chunk's K and V rows are loaded into registers
// while the current chunk is computed.
template <int D, int C, class TB>
__global__ __launch_bounds__(64 * f32_waves(D)) __attribute__((amdgpu_waves_per_eu(D * C <= 4096 ? 3 : (f32_waves(D) == 8 ? 2 : 1)))) void causal_f32(
    CausalArgs a, TB tb) {  // three workgroups per CU where the LDS allows (d = 64, 64-token chunks)
  constexpr int NW = f32_waves(D);   // waves: 8 at d = 128 (one workgroup per CU fits the LDS)
  constexpr int NT = 64 * NW;
  constexpr int LD = D + 4;
  constexpr int NI = C / 16;         // token tiles per chunk
  constexpr int NA = D / 16;         // feature tiles
  constexpr int NC = D / 16;         // output column tiles
  constexpr int NCW = NC / NW;       // state column tiles per wave
  constexpr int KM = D / 16;         // 16-feature groups of a reduction over features
  constexpr int SH = NI >= NW ? 1 : NW / NI;  // waves sharing a query tile (splitting its columns)
  constexpr int TPW = NI >= NW ? NI / NW : 1; // query tiles per wave
  constexpr int NCO = NC / SH;       // output column tiles per wave
  constexpr int PPR = D / 4;         // 16-byte pieces per row
  constexpr int NP = C * PPR / NT;   // K (and V) pieces per thread
  static_assert((NI == 8 || NI == 4) && NCW >= 1 && SH <= 2 && NP >= 1, "chunk");
  __shared__ __attribute__((aligned(16))) float Kn[C * LD];
  __shared__ __attribute__((aligned(16))) float Vn[C * LD];
  __shared__ __attribute__((aligned(16))) float St[D * LD];  // S^T of the state before the chunk
  __shared__ float zf[D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.x / a.segs, seg = blockIdx.x % a.segs;
  const HeadSpan sp = head_span(tb, a.n, bh);
  const int64_t t0 = seg * a.seg_len;
  if (t0 >= sp.n) return;  // a segment past a shorter sequence's end (variable lengths)
  const int64_t t1 = t0 + a.seg_len < sp.n ? t0 + a.seg_len : sp.n;
  const float* Q = reinterpret_cast<const float*>(a.q) + sp.row0 * D;
  const float* K = reinterpret_cast<const float*>(a.k) + sp.row0 * D;
  const float* V = reinterpret_cast<const float*>(a.v) + sp.row0 * D;
  float* O = reinterpret_cast<float*>(a.out) + sp.row0 * D;

  f32x4 accS[NA][NCW];
#pragma unroll
  for (int at = 0; at < NA; ++at)
#pragma unroll
    for (int p = 0; p < NCW; ++p) accS[at][p] = zero4();
  float zinit = 0.f;
  if (a.s0) {  // the state before the sequence
    const float* s0 = a.s0 + bh * D * D;
#pragma unroll
    for (int at = 0; at < NA; ++at)
#pragma unroll
      for (int p = 0; p < NCW; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) accS[at][p][r] = s0[(at * 16 + g * 4 + r) * D + (wave + NW * p) * 16 + l16];
    if (tid < D) zinit = a.z0[bh * D + tid];
  }
  for (int64_t s = 0; s < seg; ++s) {      // same grouping as in the bf16 kernel
    f32x4 part[NA][NCW];
    float zpart = 0.f;
#pragma unroll
    for (int at = 0; at < NA; ++at)
#pragma unroll
      for (int p = 0; p < NCW; ++p) part[at][p] = zero4();
    for (int64_t q = 0; q < a.seg_parts; ++q) {
      const float* st = seg_state_ptr(a, bh, s * a.seg_parts + q, D);
#pragma unroll
      for (int at = 0; at < NA; ++at)
#pragma unroll
        for (int p = 0; p < NCW; ++p)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            part[at][p][r] += st[(at * 16 + g * 4 + r) * D + (wave + NW * p) * 16 + l16];
      if (tid < D) zpart += st[D * D + tid];
    }
#pragma unroll
    for (int at = 0; at < NA; ++at)
#pragma unroll
      for (int p = 0; p < NCW; ++p) accS[at][p] += part[at][p];
    zinit += zpart;
  }
  if (tid < D) zf[tid] = zinit;

  // The key sums z are added on the vector ALU beside the state update (whose MFMA pipe is the
  // busy one), each wave for feature tiles wave + NW i: lane (l16, g) sums the keys 4 ks + g of
  // feature 16 (wave + NW i) + l16 over the chunk, the four lane groups are summed once, and zf
  // takes the chunk's sums for the next chunk's normalisers.
  constexpr int NZW = NA / NW;

  // S^T of the initial state for the first chunk's inter-chunk product
  auto write_st = [&]() {
#pragma unroll
    for (int at = 0; at < NA; ++at)
#pragma unroll
      for (int p = 0; p < NCW; ++p)
        *reinterpret_cast<f32x4*>(&St[((wave + NW * p) * 16 + l16) * LD + at * 16 + g * 4]) = accS[at][p];
  };
  write_st();
  __syncthreads();  // zf holds the initial key sums

  // K and V pieces: piece tid + NT p of a chunk is row (tid / PPR) + (NT / PPR) p, columns
  // 4 (tid % PPR) .. + 3.  Rows past the segment end read row t1 - 1 and are zeroed in LDS.
  auto prow = [&](int p) { return tid / PPR + p * (NT / PPR); };
  // the query tile of this wave's tp-th share, and the first of its output column tiles: with
  // four waves, tiles w and NI - 1 - w (NI = 8) or w (NI = 4), all columns; with eight waves
  // and four tiles, tile w shared by waves w and 7 - w, which take half the columns each (a SIMD
  // holds waves s and s + 4, so tiles s and 3 - s: the causal triangle is balanced per SIMD)
  auto tile_of = [&](int tp) { return SH == 1 ? (tp == 0 ? wave : NI - 1 - wave) : (wave < 4 ? wave : 7 - wave); };
  const int cb = SH == 1 ? 0 : (wave < 4 ? 0 : NCO);
  const int pcol = (tid % PPR) * 4;
  f32x4 kq[NP], vq[NP];
  auto load_kv = [&](int64_t c0) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int64_t r = c0 + prow(p) < t1 ? c0 + prow(p) : t1 - 1;
      kq[p] = *reinterpret_cast<const f32x4*>(K + r * D + pcol);
      vq[p] = *reinterpret_cast<const f32x4*>(V + r * D + pcol);
    }
  };
  load_kv(t0);
  for (int64_t c0 = t0; c0 < t1; c0 += C) {
    // this wave's query rows (rows past the end read row t1 - 1; their outputs are not stored)
    f32x4 qv[TPW][KM];
#pragma unroll
    for (int tp = 0; tp < TPW; ++tp) {
      const int it = tile_of(tp);
      const int64_t row = c0 + it * 16 + l16;
      const int64_t r = row < t1 ? row : t1 - 1;
#pragma unroll
      for (int m = 0; m < KM; ++m) qv[tp][m] = *reinterpret_cast<const f32x4*>(Q + r * D + m * 16 + g * 4);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {  // phi on K; rows past the end are zero in both tiles
      const bool ok = c0 + prow(p) < t1;
      f32x4 kk = kq[p];
      kk.x = phi(kk.x);
      kk.y = phi(kk.y);
      kk.z = phi(kk.z);
      kk.w = phi(kk.w);
      *reinterpret_cast<u32x4*>(&Kn[prow(p) * LD + pcol]) = keep_if(__builtin_bit_cast(u32x4, kk), ok);
      *reinterpret_cast<u32x4*>(&Vn[prow(p) * LD + pcol]) = keep_if(__builtin_bit_cast(u32x4, vq[p]), ok);
    }
    __syncthreads();  // tiles, S^T and z of this chunk ready
    load_kv(c0 + C);  // the next chunk's rows arrive while this one is computed

#pragma unroll
    for (int tp = 0; tp < TPW; ++tp) {
      const int it = tile_of(tp);
      f32x4 qf[KM];
      float dpart = 0.f;  // phi(q) . z over this lane's features
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        qf[m].x = phi(qv[tp][m].x);
        qf[m].y = phi(qv[tp][m].y);
        qf[m].z = phi(qv[tp][m].z);
        qf[m].w = phi(qv[tp][m].w);
        dpart += qf[m].x * zf[m * 16 + g * 4] + qf[m].y * zf[m * 16 + g * 4 + 1] +
                 qf[m].z * zf[m * 16 + g * 4 + 2] + qf[m].w * zf[m * 16 + g * 4 + 3];
      }
      f32x4 acco[NCO];
#pragma unroll
      for (int c = 0; c < NCO; ++c) acco[c] = zero4();
      // inter-chunk: S^T phi(Q)^T (this wave's output columns)
#pragma unroll
      for (int m = 0; m < KM; ++m)
#pragma unroll
        for (int c = 0; c < NCO; ++c) {
          const f32x4 sv = *reinterpret_cast<const f32x4*>(&St[((cb + c) * 16 + l16) * LD + m * 16 + g * 4]);
          acco[c] = mfma_f32(sv.x, qf[m].x, acco[c]);
          acco[c] = mfma_f32(sv.y, qf[m].y, acco[c]);
          acco[c] = mfma_f32(sv.z, qf[m].z, acco[c]);
          acco[c] = mfma_f32(sv.w, qf[m].w, acco[c]);
        }
      // intra-chunk, one key tile at a time: A^T = phi(K_jt) phi(Q_it)^T (masked on the
      // diagonal tile), then V^T A^T; the key sums 1^T A^T go into this lane's part of the
      // denominator (its rows 4g..4g+3 of the tile), summed over the lane groups once per row
      for (int jt = 0; jt <= it; ++jt) {
        f32x4 accA = zero4();
#pragma unroll
        for (int m = 0; m < KM; ++m) {
          const f32x4 kf = *reinterpret_cast<const f32x4*>(&Kn[(jt * 16 + l16) * LD + m * 16 + g * 4]);
          accA = mfma_f32(kf.x, qf[m].x, accA);
          accA = mfma_f32(kf.y, qf[m].y, accA);
          accA = mfma_f32(kf.z, qf[m].z, accA);
          accA = mfma_f32(kf.w, qf[m].w, accA);
        }
        if (jt == it) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (g * 4 + r > l16) accA[r] = 0.f;
        }
        dpart += (accA[0] + accA[1]) + (accA[2] + accA[3]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = jt * 16 + g * 4 + r;
#pragma unroll
          for (int c = 0; c < NCO; ++c) acco[c] = mfma_f32(Vn[j * LD + (cb + c) * 16 + l16], accA[r], acco[c]);
        }
      }
      const float den = sum_over_groups(dpart);
      const int64_t row = c0 + it * 16 + l16;
      if (row < t1) {
        // one IEEE division per row, then products (within 1.5 ulp of a division per element);
        // a denominator too small for its reciprocal to be finite keeps the exact divisions
        const float inv = 1.0f / den;
        const bool tiny = !(den >= 0x1p-120f);
#pragma unroll
        for (int c = 0; c < NCO; ++c) {
          f32x4 o = {acco[c][0] * inv, acco[c][1] * inv, acco[c][2] * inv, acco[c][3] * inv};
          if (tiny) o = f32x4{acco[c][0] / den, acco[c][1] / den, acco[c][2] / den, acco[c][3] / den};
          *reinterpret_cast<f32x4*>(O + row * D + (cb + c) * 16 + g * 4) = o;
        }
      }
    }
    __syncthreads();  // S^T, z and the tiles are no longer read for outputs

    // state update: S[:, own cols] += phi(K)^T V, z[own feature tiles] += phi(K)^T 1
    float zs[NZW];
#pragma unroll
    for (int i = 0; i < NZW; ++i) zs[i] = 0.f;
    for (int ks = 0; ks < C / 4; ++ks) {
#pragma unroll
      for (int at = 0; at < NA; ++at) {
        const float ak = Kn[(ks * 4 + g) * LD + at * 16 + l16];
#pragma unroll
        for (int p = 0; p < NCW; ++p)
          accS[at][p] = mfma_f32(ak, Vn[(ks * 4 + g) * LD + (wave + NW * p) * 16 + l16], accS[at][p]);
      }
#pragma unroll
      for (int i = 0; i < NZW; ++i) zs[i] += Kn[(ks * 4 + g) * LD + (wave + NW * i) * 16 + l16];
    }
#pragma unroll
    for (int i = 0; i < NZW; ++i) {
      const float zc = sum_over_groups(zs[i]);
      if (g == 0) zf[(wave + NW * i) * 16 + l16] += zc;
    }
    write_st();
    __syncthreads();  // before the next chunk overwrites the tiles
  }

  // the state after the last token, from the last segment's workgroup
  if (a.sn && seg == (sp.n - 1) / a.seg_len) {
    float* sn = a.sn + bh * D * D;
#pragma unroll
    for (int at = 0; at < NA; ++at)
#pragma unroll
      for (int p = 0; p < NCW; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) sn[(at * 16 + g * 4 + r) * D + (wave + NW * p) * 16 + l16] = accS[at][p][r];
    if (tid < D) a.zn[bh * D + tid] = zf[tid];
  }
}

// The final state of an empty sequence is the initial one: sn, zn = s0, z0 (or zeros).  One
// float4 per thread, grid-stride over all heads.
template <int D>
__global__ __launch_bounds__(256) void state_copy(CausalArgs a) {
  constexpr int64_t S4 = D * D / 4, Z4 = D / 4;
  const int64_t total = a.bh * (S4 + Z4);
  for (int64_t e = blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    if (e < a.bh * S4) {
      reinterpret_cast<f32x4*>(a.sn)[e] = a.s0 ? reinterpret_cast<const f32x4*>(a.s0)[e] : zero4();
    } else {
      const int64_t f = e - a.bh * S4;
      reinterpret_cast<f32x4*>(a.zn)[f] = a.z0 ? reinterpret_cast<const f32x4*>(a.z0)[f] : zero4();
    }
  }
}

hipError_t launch_state_copy(const CausalArgs& a, int d, hipStream_t s) {
  const int64_t total = a.bh * (d * d + d) / 4;
  const int64_t blocks = total / 256 + 1 < 4096 ? total / 256 + 1 : 4096;
  if (d == 64)
    hipLaunchKernelGGL(state_copy<64>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(state_copy<128>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, int C, class TB>
static hipError_t launch_causal_tb(const CausalArgs& a, int dtype, hipStream_t s, const TB& tb) {
  const unsigned blocks = (unsigned)(a.bh * a.segs);
  if (dtype == 1) {
    hipLaunchKernelGGL((causal_bf16<D, C, TB>), dim3(blocks), dim3(512), 0, s, a, tb);
  } else {
    if constexpr (D * C <= 8192)
      hipLaunchKernelGGL((causal_f32<D, C, TB>), dim3(blocks), dim3(64 * f32_waves(D)), 0, s, a, tb);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int C>
static hipError_t launch_causal_t(const CausalArgs& a, int dtype, hipStream_t s, const SeqTable* tab) {
  return tab ? launch_causal_tb<D, C>(a, dtype, s, *tab) : launch_causal_tb<D, C>(a, dtype, s, NoTable{});
}

hipError_t launch_causal(const CausalArgs& a, int d, int chunk, int dtype, hipStream_t s, const SeqTable* tab) {
  if (d == 64) return chunk == 64 ? launch_causal_t<64, 64>(a, dtype, s, tab) : launch_causal_t<64, 128>(a, dtype, s, tab);
  return chunk == 64 ? launch_causal_t<128, 64>(a, dtype, s, tab) : launch_causal_t<128, 128>(a, dtype, s, tab);
}

}  // namespace la
