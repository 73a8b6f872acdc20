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

// fp32 kernel: the bf16 kernel's schedule, tiles and operand layouts, with every product of fp32
// values taken on the bf16 MFMA from two-term splits (split4 / split8 / mfma_split in
// la_common.h): phi(K), V, the state S^T and z are held in LDS as two bf16 planes (hi, lo),
// phi(Q) and the masked weights A as hi and lo operands in registers, and each 16x16x32 product
// becomes four.  The running state, z, every accumulation and the output division stay fp32.
// (The fp32 MFMA, 16x16x4, does the same work at 1/16 of the bf16 rate; four terms cost 1/4 plus
// the vector work of splitting, which leaves the kernel bound by memory, not the matrix pipe.)
//
// LDS, bf16 planes: KnH/KnL [C][D + 16] phi(K); VnH/VnL [C][D] V, pieces permuted as in the bf16
// kernel (one buffer: the next chunk's V is stored after the chunk's second barrier, with K);
// StH/StL [D][D] S^T (pswz); Zr [16][D + 16], rows 0 and 1 the hi and lo of z.  d = 128 with
// 64-token chunks takes 137 KB (one workgroup per CU); d = 64 takes 55 KB with 64-token chunks
// (two per CU) and 91 KB with 128.
template <int D, int C, class TB>
__global__ __launch_bounds__(512) void causal_f32(
    CausalArgs a, TB tb) {
  constexpr int NT = 512;
  constexpr int LDK = D + 16;
  constexpr int NI = C / 16;
  constexpr int NC = D / 16;
  constexpr int NA = D / 16;
  constexpr int NAW = NA / 4;
  constexpr int NCW = NC / 2;
  constexpr int OCT = NI == 8 ? NC : NC / 2;
  constexpr int KA = D / 32;
  constexpr int KJ = C / 32;
  constexpr int PPR = D / 4;          // 16-byte fp32 pieces per row
  constexpr int RPK = C * PPR / NT;   // K (and V) pieces per thread
  static_assert(NI == 8 || NI == 4, "chunk");
  static_assert(RPK >= 1, "tile split");

  __shared__ __attribute__((aligned(16))) uint16_t KnH[C * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t KnL[C * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t VnH[C * D];
  __shared__ __attribute__((aligned(16))) uint16_t VnL[C * D];
  __shared__ __attribute__((aligned(16))) uint16_t StH[D * D];
  __shared__ __attribute__((aligned(16))) uint16_t StL[D * D];
  __shared__ __attribute__((aligned(16))) uint16_t Zr[16 * LDK];
  __shared__ float zf[D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int64_t bh = blockIdx.x / a.segs, seg = blockIdx.x % a.segs;
  const HeadSpan sp = head_span(tb, a.n, bh);
  const int64_t t0 = seg * a.seg_len;
  if (t0 >= sp.n) return;  // a segment past a shorter sequence's end (variable lengths)
  const int64_t t1 = t0 + a.seg_len < sp.n ? t0 + a.seg_len : sp.n;
  const float* Q = reinterpret_cast<const float*>(a.q) + sp.row0 * D;
  const float* K = reinterpret_cast<const float*>(a.k) + sp.row0 * D;
  const float* V = reinterpret_cast<const float*>(a.v) + sp.row0 * D;
  float* O = reinterpret_cast<float*>(a.out) + sp.row0 * D;

  const int it = wave < 4 ? wave : (NI == 8 ? 11 - wave : 7 - wave);   // this wave's query tile
  const int oc0 = (NI == 8 || wave < 4) ? 0 : NC / 2;                 // its first output column tile
  const int sa0 = NAW * (wave & 3), sc0 = NCW * (wave >> 2);           // its state block
  const bool zown = wave < 4;                                          // keeps z of tiles sa0..

  // ---- initial state: sum of the leading segments' sums (the bf16 kernel's grouping)
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
  auto write_state = [&]() {
#pragma unroll
    for (int i = 0; i < NAW; ++i)
#pragma unroll
      for (int j = 0; j < NCW; ++j) {
        u32x2 h, l;
        split4(accS[i][j], h, l);
        const int o = pswz<D>((sc0 + j) * 16 + l16, (sa0 + i) * 16 + g * 4);
        *reinterpret_cast<u32x2*>(&StH[o]) = h;
        *reinterpret_cast<u32x2*>(&StL[o]) = l;
      }
  };
  write_state();
  __syncthreads();
  const uint32_t one2 = 0x3F803F80u;  // two bf16 ones
  u32x4 ones;                          // A operand with a row of ones (row 0)
  ones.x = ones.y = ones.z = ones.w = (l16 == 0) ? one2 : 0u;
  f32x4 accz[NAW];                     // z of this wave's feature tiles (column 0 of phi(K)^T ones)
  const u32x4 zones = zown ? ones : zero_u4();
#pragma unroll
  for (int i = 0; i < NAW; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) accz[i][r] = (zown && l16 == 0) ? zf[(sa0 + i) * 16 + g * 4 + r] : 0.f;
  for (int e = tid; e < 16 * D; e += NT) {
    const int row = e / D, c = e % D;
    uint16_t val = 0;
    if (row == 0) val = (uint16_t)(__float_as_uint(zf[c]) >> 16);
    if (row == 1) val = __builtin_bit_cast(uint16_t, (__bf16)split_rest(zf[c]));
    Zr[row * LDK + c] = val;
  }

  // ---- K and V tiles: fp32 piece tid + 512 p of each (16-byte pieces, row-major)
  f32x4 kq[RPK], vq[RPK];
  f32x4 qr[KA][2];  // this wave's query rows (raw): features 32 ks + 8 g .. + 7
  u32x2 khi[RPK], klo[RPK], vhi[RPK], vlo[RPK];
  auto prow = [&](int p) { return tid / PPR + p * (NT / PPR); };
  const int pcol = (tid % PPR) * 4;
  auto ldf = [&](const float* base, int64_t row, int col) {  // rows past the end read row t1 - 1
    const int64_t r = row < t1 ? row : t1 - 1;
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(base + r * D + col));
  };
  auto load_k = [&](int64_t c0) {
#pragma unroll
    for (int p = 0; p < RPK; ++p) kq[p] = ldf(K, c0 + prow(p), pcol);
  };
  auto load_v = [&](int64_t c0) {
#pragma unroll
    for (int p = 0; p < RPK; ++p) vq[p] = ldf(V, c0 + prow(p), pcol);
  };
  auto load_q = [&](int64_t c0) {  // rows >= t1 are never stored
    const int64_t row = c0 + it * 16 + l16;
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) {
      qr[ks][0] = ldf(Q, row, ks * 32 + g * 8);
      qr[ks][1] = ldf(Q, row, ks * 32 + g * 8 + 4);
    }
  };
  // feature map on K, then both tiles split; rows past the segment end become zero.  V is
  // canonicalised first so that a signalling NaN stays NaN in hi.
  auto prep_kv = [&](int64_t c0) {
#pragma unroll
    for (int p = 0; p < RPK; ++p) {
      const uint32_t m = 0u - (uint32_t)(c0 + prow(p) < t1);
      f32x4 kk = kq[p], vv = vq[p];
      kk.x = phi(kk.x);
      kk.y = phi(kk.y);
      kk.z = phi(kk.z);
      kk.w = phi(kk.w);
      vv.x = __builtin_canonicalizef(vv.x);
      vv.y = __builtin_canonicalizef(vv.y);
      vv.z = __builtin_canonicalizef(vv.z);
      vv.w = __builtin_canonicalizef(vv.w);
      split4(kk, khi[p], klo[p]);
      split4(vv, vhi[p], vlo[p]);
      khi[p].x &= m;
      khi[p].y &= m;
      klo[p].x &= m;
      klo[p].y &= m;
      vhi[p].x &= m;
      vhi[p].y &= m;
      vlo[p].x &= m;
      vlo[p].y &= m;
    }
  };

  // V pieces permuted by the row as in the bf16 kernel (conflict-free transpose reads)
  constexpr int VRL = 128 / D;
  auto vofs = [&](int r, int c) { return r * D + ((((c >> 3) ^ (2 * ((r / VRL) % (D / 16))))) << 3) + (c & 7); };
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
  auto store_kv = [&]() {
#pragma unroll
    for (int p = 0; p < RPK; ++p) {
      *reinterpret_cast<u32x2*>(&KnH[prow(p) * LDK + pcol]) = khi[p];
      *reinterpret_cast<u32x2*>(&KnL[prow(p) * LDK + pcol]) = klo[p];
      *reinterpret_cast<u32x2*>(&VnH[vofs(prow(p), pcol)]) = vhi[p];
      *reinterpret_cast<u32x2*>(&VnL[vofs(prow(p), pcol)]) = vlo[p];
    }
  };

  load_k(t0);
  load_v(t0);
  load_q(t0);
  prep_kv(t0);
  store_kv();
  for (int64_t c0 = t0; c0 < t1; c0 += C) {
    __syncthreads();  // tiles of this chunk, S^T and Zr ready
    // next chunk's loads in three groups, as in the bf16 kernel
    __builtin_amdgcn_sched_barrier(0);
    load_k(c0 + C);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 qh[KA], ql[KA];
    auto split_q = [&]() {
#pragma unroll
      for (int ks = 0; ks < KA; ++ks) {
        f32x4 x0 = qr[ks][0], x1 = qr[ks][1];
        x0.x = phi(x0.x);
        x0.y = phi(x0.y);
        x0.z = phi(x0.z);
        x0.w = phi(x0.w);
        x1.x = phi(x1.x);
        x1.y = phi(x1.y);
        x1.z = phi(x1.z);
        x1.w = phi(x1.w);
        split8(x0, x1, qh[ks], ql[ks]);
      }
    };

    // ---- state update in registers: S[own block] += phi(K_c)^T V_c ; z
    auto update_state = [&]() {
#pragma unroll
    for (int ks = 0; ks < KJ; ++ks) {
      u32x4 akh[NAW], akl[NAW];
#pragma unroll
      for (int i = 0; i < NAW; ++i) {
        akh[i] = ld_rows_operand(KnH, LDK, ks * 32, (sa0 + i) * 16, l16, g);
        akl[i] = ld_rows_operand(KnL, LDK, ks * 32, (sa0 + i) * 16, l16, g);
        accz[i] = mfma_bf16(akl[i], zones, accz[i]);  // zones is zero where z is not kept
        accz[i] = mfma_bf16(akh[i], zones, accz[i]);
      }
#pragma unroll
      for (int j = 0; j < NCW; ++j) {
        const u32x4 bvh = ld_v_operand(VnH, ks * 32, (sc0 + j) * 16);
        const u32x4 bvl = ld_v_operand(VnL, ks * 32, (sc0 + j) * 16);
#pragma unroll
        for (int i = 0; i < NAW; ++i) accS[i][j] = mfma_split(akh[i], akl[i], bvh, bvl, accS[i][j]);
      }
    }
    };
    // Waves 0..3 update the state here, waves 4..7 (the other wave of each SIMD) after their
    // outputs, where it runs on the matrix pipe beside the first wave's vector work (output
    // scaling, the next chunk's feature map and splits)
    split_q();
    if (wave_u < 4) update_state();
    __builtin_amdgcn_sched_barrier(0);
    load_v(c0 + C);
    __builtin_amdgcn_sched_barrier(0);

    // ---- this wave's query tile: inter-chunk part S^T phi(Q)^T and [z_hi; z_lo] phi(Q)^T
    f32x4 acco[OCT];
    f32x4 accd = zero4();
#pragma unroll
    for (int ct = 0; ct < OCT; ++ct) acco[ct] = zero4();
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) {
#pragma unroll
      for (int ct = 0; ct < OCT; ++ct) {
        const int o = pswz<D>((oc0 + ct) * 16 + l16, ks * 32 + g * 8);
        acco[ct] = mfma_split(ld16(&StH[o]), ld16(&StL[o]), qh[ks], ql[ks], acco[ct]);
      }
      const u32x4 zr = ld16(&Zr[l16 * LDK + ks * 32 + g * 8]);
      accd = mfma_bf16(zr, ql[ks], accd);
      accd = mfma_bf16(zr, qh[ks], accd);
    }
    // intra-chunk: A^T = phi(K) phi(Q)^T masked to key <= query, split, then V^T A^T and
    // ones A^T; step m covers key tiles 2m and 2m + 1, and the A^T products of step m + 1 go out
    // before the V products of step m (the bf16 kernel's pipeline)
    auto a_tiles = [&](int m, f32x4& a0, f32x4& a1) {
      a0 = zero4();
      a1 = zero4();
#pragma unroll
      for (int ks = 0; ks < KA; ++ks) {
        const int o0 = (2 * m * 16 + l16) * LDK + ks * 32 + g * 8, o1 = o0 + 16 * LDK;
        a0 = mfma_split(ld16(&KnH[o0]), ld16(&KnL[o0]), qh[ks], ql[ks], a0);
        a1 = mfma_split(ld16(&KnH[o1]), ld16(&KnL[o1]), qh[ks], ql[ks], a1);
      }
    };
    auto split_a = [&](int m, f32x4 a0, f32x4 a1, u32x4& ah, u32x4& al) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (2 * m == it && g * 4 + r > l16) a0[r] = 0.f;
        if (2 * m + 1 > it || (2 * m + 1 == it && g * 4 + r > l16)) a1[r] = 0.f;
      }
      split8(a0, a1, ah, al);
    };
    auto av_step = [&](int m, u32x4 ah, u32x4 al) {
#pragma unroll
      for (int ct = 0; ct < OCT; ++ct)
        acco[ct] = mfma_split(ld_v_operand(VnH, m * 32, (oc0 + ct) * 16), ld_v_operand(VnL, m * 32, (oc0 + ct) * 16),
                         ah, al, acco[ct]);
      accd = mfma_bf16(ones, al, accd);
      accd = mfma_bf16(ones, ah, accd);
    };
    const int mlast = it >> 1;
    f32x4 a0, a1;
    a_tiles(0, a0, a1);
#pragma unroll
    for (int m = 0; m < NI / 2 - 1; ++m) {
      if (m < mlast) {
        u32x4 ah, al;
        split_a(m, a0, a1, ah, al);
        a_tiles(m + 1, a0, a1);
        av_step(m, ah, al);
      }
    }
    u32x4 ah, al;
    split_a(mlast, a0, a1, ah, al);
    av_step(mlast, ah, al);

    const float den = __shfl(accd[0] + accd[1], l16);
    const int64_t row = c0 + it * 16 + l16;
    if (row < t1) {
      // one IEEE division per row, then products (within 1.5 ulp of a division per element);
      // a denominator too small for its reciprocal to be finite keeps the exact divisions
      const float inv = 1.0f / den;
      const bool tiny = !(den >= 0x1p-120f);
#pragma unroll
      for (int ct = 0; ct < OCT; ++ct) {
        f32x4 o = {acco[ct][0] * inv, acco[ct][1] * inv, acco[ct][2] * inv, acco[ct][3] * inv};
        if (tiny) o = f32x4{acco[ct][0] / den, acco[ct][1] / den, acco[ct][2] / den, acco[ct][3] / den};
        *reinterpret_cast<f32x4*>(O + row * D + (oc0 + ct) * 16 + g * 4) = o;
      }
    }
    if (wave_u >= 4) update_state();
    __builtin_amdgcn_sched_barrier(0);
    load_q(c0 + C);
    __builtin_amdgcn_sched_barrier(0);
    prep_kv(c0 + C);  // past the last chunk these are zero tiles that nothing reads
    __syncthreads();  // every wave is done reading this chunk's tiles, S^T and Zr

    // ---- the next chunk's tiles, the new state
    store_kv();
    write_state();
    if (zown && l16 == 0) {
#pragma unroll
      for (int i = 0; i < NAW; ++i) {
        u32x2 h, l;
        split4(accz[i], h, l);
        *reinterpret_cast<u32x2*>(&Zr[(sa0 + i) * 16 + g * 4]) = h;
        *reinterpret_cast<u32x2*>(&Zr[LDK + (sa0 + i) * 16 + g * 4]) = l;
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
      hipLaunchKernelGGL((causal_f32<D, C, TB>), dim3(blocks), dim3(512), 0, s, a, tb);
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
