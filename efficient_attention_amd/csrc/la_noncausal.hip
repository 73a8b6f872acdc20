// la_noncausal.hip -- non-causal linear attention on gfx950, and the per-block state sums that
// the causal path reuses.
//
// Math ("Efficient Transformers: Linear Attention and Flash Attention", section "Linear
// attention: reordering the matmuls, not shrinking them", eq. Attention_i):
//     KV = sum_j phi(k_j) v_j^T  (D x d),  z = sum_j phi(k_j)  (D),
//     out_i = phi(q_i) KV / phi(q_i) z.
// Because the sums split over any partition of the keys (associativity, section "Worked
// example"), stage 1 sums slices of keys in parallel into per-slice partials; whoever needs a
// group's state adds its slices in a fixed order (deterministic, no float atomics): the
// output kernel's prologue, state_reduce, or the causal kernel's prologue.  Stage 2 streams
// the queries.
//
// Kernels
//   kv_state_*   stage 1.  Grid = groups x slices (1-D).  A group is a contiguous token range
//                of one head; its result, [KV (D x D) | z (D)] fp32, lands in `state[group]`.
//   nc_out_*     stage 2.  Grid = heads x query tiles (1-D).
#include "la_common.h"
#include "la_kernels.h"

namespace la {

__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// ----------------------------------------------------------------------------- stage 1
// Group bookkeeping shared by the bf16 and fp32 variants.
struct GroupRange {
  int64_t g, bh, s;   // group, head, slice
  int64_t row0, hn;   // the head's first row and its tokens
  int64_t t0, t1;     // token range [t0, t1) of this slice within the head
};

// A slice past its head's end is empty (t0 >= t1); its workgroup still writes a zero partial,
// reading only row hn - 1 (a head without tokens has no workgroup that reads anything).
template <class TB>
__device__ __forceinline__ GroupRange group_range(const KvStateArgs& a, const TB& tb) {
  GroupRange r;
  r.g = blockIdx.x / a.slices;
  r.s = blockIdx.x % a.slices;
  r.bh = r.g / a.groups_per_head;
  const HeadSpan sp = head_span(tb, a.n, r.bh);
  r.row0 = sp.row0;
  r.hn = sp.n;
  int64_t seg = r.g % a.groups_per_head;
  int64_t gs = seg * a.group_len;
  int64_t ge = gs + a.group_len < sp.n ? gs + a.group_len : sp.n;
  r.t0 = gs + r.s * a.slice_len;
  r.t1 = r.t0 + a.slice_len < ge ? r.t0 + a.slice_len : ge;
  return r;
}

// Write this workgroup's [KV | z] (fp32, adjacent in LDS) to its slot: the group state
// when the group has one slice, otherwise the slice's partial, which state_reduce (or the
// causal kernel's prologue) adds up after this kernel has finished.  There is no cross-
// workgroup synchronisation inside the kernel: the kernel boundary orders the two steps.
template <int D>
__device__ void publish_state(const KvStateArgs& a, const GroupRange& gr, const float* kv_lds) {
  constexpr int E = D * D + D;
  constexpr int E4 = E / 4;
  static_assert(E % 4 == 0, "state size");
  const f32x4* src = reinterpret_cast<const f32x4*>(kv_lds);
  f32x4* dst = reinterpret_cast<f32x4*>(a.slices == 1 ? a.state + gr.g * E
                                                       : a.partials + (gr.g * a.slices + gr.s) * E);
  for (int e = threadIdx.x; e < E4; e += 256) dst[e] = src[e];
}

// Adds the slices' partials of every group in slice order (deterministic).  Grid: groups x
// ceil(E/4/256) workgroups of 256 threads, one float4 of the state per thread.
template <int D>
__global__ __launch_bounds__(256) void state_reduce(KvStateArgs a) {
  constexpr int E = D * D + D;
  constexpr int E4 = E / 4;
  constexpr int BPG = (E4 + 255) / 256;
  const int64_t g = blockIdx.x / BPG;
  const int e = (int)(blockIdx.x % BPG) * 256 + threadIdx.x;
  if (e >= E4) return;
  const f32x4* src = reinterpret_cast<const f32x4*>(a.partials + g * a.slices * E) + e;
  f32x4 acc = zero4();
  for (int64_t p = 0; p < a.slices; ++p) acc += src[p * E4];
  reinterpret_cast<f32x4*>(a.state + g * E)[e] = acc;
}

// Writes a wave's block of the state straight from its MFMA accumulators: rows (features)
// 16 at + 4g + r, columns 16 c + l16, and z (already summed over the lane groups) by the lanes
// of group 0.
template <int D, int NA, int NC>
__device__ __forceinline__ void store_state_block(float* dst, int at0, const f32x4 (&acc)[NA][NC],
                                                  const float (&z)[NA], int l16, int g) {
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int at = at0 + i;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(at * 16 + g * 4 + r) * D + c * 16 + l16] = acc[i][c][r];
    if (g == 0) dst[D * D + at * 16 + l16] = z[i];
  }
}

// bf16 stage 1.  Tiles of T tokens.  phi(K) and V are stored token-major in LDS, as they come
// from HBM (16 consecutive lanes load one 256-byte row when D = 128), and the MFMA operands of
// phi(K)^T V, whose reduction index is the token, are read through LDS transpose reads: no
// transposes in registers.  Wave w accumulates feature tiles NA*w.. against all value columns.
// Loads run NS - 1 tiles ahead in NS register sets (the tile loop is unrolled by NS; loads past
// the end are clamped and their rows masked, so they need no condition).  Small LDS and
// register footprints let several workgroups share a CU and overlap one another's loads,
// feature map and MFMA work.
template <int D, class TB>
__global__ __launch_bounds__(256) void kv_state_bf16(KvStateArgs a, TB tb) {
  constexpr int T = kStateTileBf16;  // tokens per tile
  constexpr int LDK = D + 16;        // row stride of 8 (mod 64) dwords x odd: conflict-free reads
  constexpr int PPR = D / 8;         // 16-byte pieces per row
  constexpr int NP = T * PPR / 256;  // pieces per thread and tensor
  constexpr int NA = D / 64;         // feature tiles per wave
  constexpr int NC = D / 16;         // value-column tiles
  constexpr int NS = D == 64 ? 3 : 2;  // register sets of loads in flight
  static_assert(NP >= 1 && T % 32 == 0, "tile");
  __shared__ __attribute__((aligned(16))) uint16_t Kn[T * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Vn[T * LDK];

  const GroupRange gr = group_range(a, tb);
  if (gr.hn == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const uint16_t* K = reinterpret_cast<const uint16_t*>(a.k) + gr.row0 * D;
  const uint16_t* V = reinterpret_cast<const uint16_t*>(a.v) + gr.row0 * D;

  f32x4 acc[NA][NC];
  float zacc[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    zacc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[i][c] = zero4();
  }

  auto prow = [&](int p) { return tid / PPR + p * (256 / PPR); };
  const int pcol = (tid % PPR) * 8;
  u32x4 kq[NS][NP], vq[NS][NP];
  auto load = [&](int64_t t0, u32x4 (&k)[NP], u32x4 (&v)[NP]) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      k[p] = ld16_clamp_nt(K, t0 + prow(p), gr.t1, D, pcol);
      v[p] = ld16_clamp_nt(V, t0 + prow(p), gr.t1, D, pcol);
    }
  };
  auto tile = [&](int64_t t0, u32x4 (&k)[NP], u32x4 (&v)[NP]) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {  // phi on K; rows past the end are zero in both tiles
      const bool ok = t0 + prow(p) < gr.t1;
      k[p] = keep_if(phi_bf16x8(k[p]), ok);
      v[p] = keep_if(v[p], ok);
    }
    __syncthreads();  // the previous tile's operands have been read
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      st16(&Kn[prow(p) * LDK + pcol], k[p]);
      st16(&Vn[prow(p) * LDK + pcol], v[p]);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < T / 32; ++s) {
      u32x4 bv[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) bv[c] = ld_rows_operand(Vn, LDK, s * 32, c * 16, l16, g);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const u32x4 ak = ld_rows_operand(Kn, LDK, s * 32, (wave * NA + i) * 16, l16, g);
        zacc[i] += sum_bf16x8(ak);
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[i][c] = mfma_bf16(ak, bv[c], acc[i][c]);
      }
    }
  };

  // The sets go out strictly in order (scheduling barriers): the compiler's wait counts for a
  // set assume the loads issued after it, and an interleaved order would make it wait for
  // later sets as well.
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    load(gr.t0 + u * T, kq[u], vq[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int64_t t0 = gr.t0; t0 < gr.t1; t0 += NS * T) {  // spare tiles past the end are all zero
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      tile(t0 + u * T, kq[u], vq[u]);
      __builtin_amdgcn_sched_barrier(0);
      load(t0 + (u + NS) * T, kq[u], vq[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  float z[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) z[i] = sum_over_groups(zacc[i]);
  float* dst = a.slices == 1 ? a.state + gr.g * (D * D + D)
                             : a.partials + (gr.g * a.slices + gr.s) * (D * D + D);
  store_state_block<D, NA, NC>(dst, wave * NA, acc, z, l16, g);
}

// bf16 stage 1 for D = 64, one wave per token stream.  Wave w of the workgroup takes tiles
// w, w + 4, ... of TW tokens; it stores phi(K) and V token-major in its own LDS area and reads
// them back as MFMA operands with transpose reads.  A wave's LDS accesses are executed in
// order, so the loop needs no barrier: waves stream independently instead of waiting for the
// slowest at every tile.  Each wave accumulates the whole 64 x 64 state (16 MFMA tiles) and z,
// phi(K)^T times a column of ones: one more MFMA per feature tile, from the same bf16 phi(K)
// operands as the state, on the MFMA pipe instead of the vector ALU (which the feature map
// keeps busy).  The four partial states are added at the end in a fixed order,
// ((w0 + w2) + (w1 + w3)).
template <int D, class TB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void kv_state_bf16_waves(KvStateArgs a, TB tb) {
  constexpr int TW = kStateTileWave;  // tokens per wave tile
  constexpr int LDK = D + 16;          // row stride of 8 (mod 64) dwords x odd: conflict-free reads
  constexpr int PPR = D / 8;           // 16-byte pieces per row
  constexpr int NP = TW * PPR / 64;    // pieces per lane and tensor
  constexpr int NT = D / 16;           // feature tiles = value-column tiles
  constexpr int NS = 2;                // register sets of loads in flight
  constexpr int WL = 2 * TW * LDK;     // LDS elements per wave
  static_assert(D == 64 && TW == 32, "one 32-token k-step per tile");
  static_assert(4 * WL * 2 >= 2 * (D * D + D) * 4, "the final combine reuses the tile areas");
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * WL];

  const GroupRange gr = group_range(a, tb);
  if (gr.hn == 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar tile addresses
  const int l16 = lane & 15, g = lane >> 4;
  const uint16_t* K = reinterpret_cast<const uint16_t*>(a.k) + gr.row0 * D;
  const uint16_t* V = reinterpret_cast<const uint16_t*>(a.v) + gr.row0 * D;
  uint16_t* Kw = lds + wave * WL;
  uint16_t* Vw = Kw + TW * LDK;

  f32x4 acc[NT][NT];
  f32x4 accz[NT];  // z of feature tile i: column 0, i.e. lanes l16 == 0, rows 4g + r
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    accz[i] = zero4();
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[i][c] = zero4();
  }
  u32x4 ones;  // B operand: a column of bf16 ones (column 0)
  ones.x = ones.y = ones.z = ones.w = l16 == 0 ? 0x3F803F80u : 0u;

  auto prow = [&](int p) { return lane / PPR + p * (64 / PPR); };
  const int pcol = (lane % PPR) * 8;
  u32x4 kq[NS][NP], vq[NS][NP];
  auto load = [&](int64_t t0, u32x4 (&k)[NP], u32x4 (&v)[NP]) {
    const TileRows tr = tile_rows(t0, gr.t1, TW);
    const uint16_t* kt = K + tr.first * D;
    const uint16_t* vt = V + tr.first * D;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      k[p] = ld16_row(kt, prow(p), tr.last, D, pcol);
      v[p] = ld16_row(vt, prow(p), tr.last, D, pcol);
    }
  };
  auto tile = [&](int64_t t0, u32x4 (&k)[NP], u32x4 (&v)[NP]) {
    const int lim = t0 < gr.t1 ? (gr.t1 - t0 < TW ? (int)(gr.t1 - t0) : TW) : 0;  // valid rows
    if (lim == TW) {  // uniform: only the last tiles need the row mask
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        st16(&Kw[prow(p) * LDK + pcol], phi_bf16x8(k[p]));
        st16(&Vw[prow(p) * LDK + pcol], v[p]);
      }
    } else {
#pragma unroll
      for (int p = 0; p < NP; ++p) {  // phi on K; rows past the end are zero in both tiles
        const bool ok = prow(p) < lim;
        st16(&Kw[prow(p) * LDK + pcol], keep_if(phi_bf16x8(k[p]), ok));
        st16(&Vw[prow(p) * LDK + pcol], keep_if(v[p], ok));
      }
    }
    u32x4 bv[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) bv[c] = ld_rows_operand(Vw, LDK, 0, c * 16, l16, g);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const u32x4 ak = ld_rows_operand(Kw, LDK, 0, i * 16, l16, g);
      accz[i] = mfma_bf16(ak, ones, accz[i]);
#pragma unroll
      for (int c = 0; c < NT; ++c) acc[i][c] = mfma_bf16(ak, bv[c], acc[i][c]);
    }
  };

  // wave tiles: t = gr.t0 + (4 j + wave) TW; loads go out strictly in order (see kv_state_bf16)
  const int64_t step = 4 * TW;
  const int64_t w0 = gr.t0 + wave * TW;
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    load(w0 + u * step, kq[u], vq[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int64_t t = w0; t - wave * TW < gr.t1; t += NS * step) {  // spare tiles are all zero
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      tile(t + u * step, kq[u], vq[u]);
      __builtin_amdgcn_sched_barrier(0);
      load(t + (u + NS) * step, kq[u], vq[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- combine the four partial states: ((w0 + w2) + (w1 + w3))
  float* xf = reinterpret_cast<float*>(lds);  // two slots of [KV | z] fp32
  constexpr int E = D * D + D;
  auto put = [&](float* slot) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) slot[(i * 16 + g * 4 + r) * D + c * 16 + l16] = acc[i][c][r];
      if (l16 == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) slot[D * D + i * 16 + g * 4 + r] = accz[i][r];
      }
    }
  };
  auto add = [&](const float* slot) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][c][r] += slot[(i * 16 + g * 4 + r) * D + c * 16 + l16];
#pragma unroll
      for (int r = 0; r < 4; ++r) accz[i][r] += slot[D * D + i * 16 + g * 4 + r];
    }
  };
  __syncthreads();  // every wave is done with its tile area
  if (wave >= 2) put(xf + (wave - 2) * E);
  __syncthreads();
  if (wave < 2) add(xf + wave * E);
  __syncthreads();
  if (wave == 1) put(xf);
  __syncthreads();
  if (wave == 0) {
    add(xf);
    float* dst = a.slices == 1 ? a.state + gr.g * E : a.partials + (gr.g * a.slices + gr.s) * E;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(i * 16 + g * 4 + r) * D + c * 16 + l16] = acc[i][c][r];
      if (l16 == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[D * D + i * 16 + g * 4 + r] = accz[i][r];
      }
    }
  }
}

// fp32 stage 1: the bf16 stage-1 layout (phi(K) and V token-major in LDS, operands of
// phi(K)^T V through transpose reads) with each tile held as two bf16 planes, hi and lo, and
// every product taken from the two-term splits on the bf16 MFMA (split4, mfma_split in
// la_common.h); accumulation is fp32.  z is the column sum of hi + lo.  The next tile's rows are loaded into registers while
// the current one is multiplied (unconditional loads, rows past the slice end clamped and then
// zeroed).  LDS: 72 KB at D = 128 (two workgroups per CU), 40 KB at D = 64 (four).
template <int D, class TB>
__global__ __launch_bounds__(256) void kv_state_f32(KvStateArgs a, TB tb) {
  constexpr int T = 64;
  constexpr int LDK = D + 16;           // row stride of 8 (mod 64) dwords x odd: conflict-free reads
  constexpr int PPR = D / 4;            // 16-byte fp32 pieces per row
  constexpr int NP = T * PPR / 256;     // pieces per thread and tensor
  constexpr int NA = D / 64;            // feature tiles per wave
  constexpr int NC = D / 16;            // value-column tiles
  __shared__ __attribute__((aligned(16))) uint16_t KnH[T * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t KnL[T * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t VnH[T * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t VnL[T * LDK];

  const GroupRange gr = group_range(a, tb);
  if (gr.hn == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const float* K = reinterpret_cast<const float*>(a.k) + gr.row0 * D;
  const float* V = reinterpret_cast<const float*>(a.v) + gr.row0 * D;

  f32x4 acc[NA][NC];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[i][c] = zero4();
  f32x4 zp = zero4();  // sums of phi(K) over this thread's rows, columns pcol .. pcol + 3
  auto prow = [&](int p) { return tid / PPR + p * (256 / PPR); };
  const int pcol = (tid % PPR) * 4;
  f32x4 kq[NP], vq[NP];
  auto load = [&](int64_t t0) {  // row t1 - 1 stands in for rows past the end (a valid row)
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int64_t r = t0 + prow(p) < gr.t1 ? t0 + prow(p) : gr.t1 - 1;
      kq[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(K + r * D + pcol));
      vq[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(V + r * D + pcol));
    }
  };
  load(gr.t0);
  for (int64_t t0 = gr.t0; t0 < gr.t1; t0 += T) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {  // phi on K, both split; rows past the end are zero
      const uint32_t m = 0u - (uint32_t)(t0 + prow(p) < gr.t1);
      f32x4 kk = kq[p], vv = vq[p];
      kk.x = phi(kk.x);
      kk.y = phi(kk.y);
      kk.z = phi(kk.z);
      kk.w = phi(kk.w);
      vv.x = __builtin_canonicalizef(vv.x);  // a signalling NaN stays NaN in hi
      vv.y = __builtin_canonicalizef(vv.y);
      vv.z = __builtin_canonicalizef(vv.z);
      vv.w = __builtin_canonicalizef(vv.w);
      zp += __builtin_bit_cast(f32x4, keep_if(__builtin_bit_cast(u32x4, kk), m != 0u));
      u32x2 kh, kl, vh, vl;
      split4(kk, kh, kl);
      split4(vv, vh, vl);
      const int o = prow(p) * LDK + pcol;
      *reinterpret_cast<u32x2*>(&KnH[o]) = u32x2{kh.x & m, kh.y & m};
      *reinterpret_cast<u32x2*>(&KnL[o]) = u32x2{kl.x & m, kl.y & m};
      *reinterpret_cast<u32x2*>(&VnH[o]) = u32x2{vh.x & m, vh.y & m};
      *reinterpret_cast<u32x2*>(&VnL[o]) = u32x2{vl.x & m, vl.y & m};
    }
    __syncthreads();
    load(t0 + T);  // the next tile arrives while this one is multiplied
#pragma unroll
    for (int s = 0; s < T / 32; ++s) {
      u32x4 akh[NA], akl[NA];
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        akh[i] = ld_rows_operand(KnH, LDK, s * 32, (wave * NA + i) * 16, l16, g);
        akl[i] = ld_rows_operand(KnL, LDK, s * 32, (wave * NA + i) * 16, l16, g);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 bvh = ld_rows_operand(VnH, LDK, s * 32, c * 16, l16, g);
        const u32x4 bvl = ld_rows_operand(VnL, LDK, s * 32, c * 16, l16, g);
#pragma unroll
        for (int i = 0; i < NA; ++i) {
          acc[i][c] = mfma_split(akh[i], akl[i], bvh, bvl, acc[i][c]);
        }
      }
    }
    __syncthreads();
  }
  // z: the 256 / PPR partial sums of each column, in thread order (the tile area is free: the
  // loop ended on a barrier)
  constexpr int ZR = 256 / PPR;
  float* zbuf = reinterpret_cast<float*>(KnH);  // [ZR][D]
  float* zfin = reinterpret_cast<float*>(VnH);  // [D]
  *reinterpret_cast<f32x4*>(&zbuf[(tid / PPR) * D + pcol]) = zp;
  __syncthreads();
  if (tid < D) {
    float zs = 0.f;
#pragma unroll
    for (int r = 0; r < ZR; ++r) zs += zbuf[r * D + tid];
    zfin[tid] = zs;
  }
  __syncthreads();
  float z[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) z[i] = zfin[(wave * NA + i) * 16 + l16];
  float* dst = a.slices == 1 ? a.state + gr.g * (D * D + D)
                             : a.partials + (gr.g * a.slices + gr.s) * (D * D + D);
  store_state_block<D, NA, NC>(dst, wave * NA, acc, z, l16, g);
}

// ----------------------------------------------------------------------------- stage 2
// The head's fp32 [KV | z] as the sum of its `slices` parts in slice order (the same order as
// state_reduce, so the sums are bitwise equal), thread tid taking float4 tid + 256 i of KV and,
// for tid < D, z[tid].  The loads of each part are all issued before they are added.
template <int D>
__device__ __forceinline__ void head_state(const NcOutArgs& a, int64_t bh, int tid,
                                           f32x4 (&kv4)[D * D / 1024], float& zv) {
  constexpr int E = D * D + D;
  constexpr int NKV4 = D * D / 1024;
  const float* base = a.state + bh * a.slices * E;
#pragma unroll
  for (int i = 0; i < NKV4; ++i) kv4[i] = zero4();
  zv = 0.f;
  for (int64_t p = 0; p < a.slices; ++p) {
    const float* st = base + p * E;
    f32x4 part[NKV4];
#pragma unroll
    for (int i = 0; i < NKV4; ++i) part[i] = reinterpret_cast<const f32x4*>(st)[tid + 256 * i];
    const float zp = tid < D ? st[D * D + tid] : 0.f;
#pragma unroll
    for (int i = 0; i < NKV4; ++i) kv4[i] += part[i];
    zv += zp;
  }
}

// bf16 output.  The workgroup turns its head's fp32 [KV | z] into bf16 MFMA operands in LDS:
// KVt[c][a] = KV[a][c], and a 16-row "normaliser" tile whose rows 0 and 1 hold z split into a
// bf16 high part and a bf16 residual (so phi(q).z keeps ~16 significant bits).  Each wave then
// takes 16 queries at a time and computes out^T = [KV^T ; z] phi(Q)^T with queries as the MFMA
// column index.
//
// HBM access is by whole rows: a wave-wide 16-byte access covers 64 / (D / 8) complete query
// rows (1 KB contiguous).  The MFMA operand, though, wants 16 queries x 32 features per access,
// so the query tile passes through a wave-private LDS tile (phi applied on the way in), and
// so does the output tile on its way out.  On this device streaming whole rows is ~8% faster
// than streaming the 64-byte row pieces the operand layout would load directly.
template <int D, class TB, int QTV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 2, D == 64 ? 4 : 2))) void nc_out_bf16(NcOutArgs a, TB tb) {
  constexpr int LD = D + 16;  // row stride of 8 mod 64 dwords: conflict-free 16-row reads
  constexpr int NC = D / 16;
  constexpr int KS = D / 32;           // MFMA k-steps
  constexpr int BB = D == 64 ? 1 : 2;  // 16-query blocks per batch and wave (see below)
  constexpr int QB = 16 * BB;          // queries per batch and wave
  constexpr int BPR = D / 8;           // 16-byte blocks per row
  constexpr int RPI = 64 / BPR;        // rows per wave-wide access
  constexpr int NL = QB / RPI;         // wave-wide accesses per batch
  constexpr int ST = QB * D;           // staging tile (QB rows x D) elements
  constexpr int64_t QT = QTV;  // queries per workgroup (nc_queries, or less when the heads are few)
  constexpr int QPW = (int)QT / 4;          // queries per wave
  __shared__ __attribute__((aligned(16))) uint16_t KVt[D * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Zr[16 * LD];
  __shared__ __attribute__((aligned(16))) uint16_t stage[4 * ST];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar tile addresses
  const int l16 = lane & 15, g = lane >> 4;
  const int prow = lane / BPR, pblk = lane % BPR;              // this lane's row / block of an access
  // Workgroups go to the 8 XCDs round-robin.  When the heads come in multiples of 8, workgroup
  // b = 8 j + x (on XCD x) takes tile j % tiles of head 8 (j / tiles) + x: all tiles of a head
  // run on one XCD, whose L2 then serves the head's partial states to all of them.  (Giving
  // each XCD a contiguous block of heads instead measured slower.)
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
  const HeadSpan sp = head_span(tb, a.n, bh);
  if (tile * QT >= sp.n) return;  // a tile past a shorter sequence's end (variable lengths)
  const int64_t n = sp.n;
  const int64_t q0 = tile * QT + wave * QB;
  const uint16_t* Q = reinterpret_cast<const uint16_t*>(a.q) + sp.row0 * D;
  uint16_t* O = reinterpret_cast<uint16_t*>(a.out) + sp.row0 * D;
  uint16_t* Ts = stage + wave * ST;  // this wave's staging tile: phi(Q) in, then the outputs

  // Staging tile layout: row r, 16-byte block b at r * D + 8 (b ^ (r & 7)) (D = 64, 8 blocks
  // per row) or 8 (b ^ (r & 15)) (D = 128).  Measured with the LDS bank-conflict counters on
  // gfx950: whole-row accesses (the HBM side) and the 16-row operand reads are conflict-free,
  // the accumulator writes (16 rows x 8 bytes) 2-way, which no permutation tried avoids.
  auto sofs = [](int r, int b) { return r * D + ((b ^ (r & (D == 64 ? 7 : 15))) << 3); };

  // Queries go in batches: in batch b the four waves take consecutive runs of QB queries.  For
  // D = 128 a batch holds two 16-query blocks, which share every KV^T operand read from LDS:
  // with one block per batch the 32 KB of KV^T would be read from LDS for every 8 KB of HBM
  // traffic.  NS register sets keep the next NS - 1 batches in flight (the loop is unrolled by
  // NS; the loads past the last batch re-read it, which costs no HBM traffic, so no load is
  // conditional).  Every workgroup starts at once and first waits for its head's state, so the
  // state is read first, ahead of the query sets in the memory queue; the first query sets then
  // load while the state is converted.
  constexpr int NBATCH = QPW / QB;
  constexpr int NS = 4;
  static_assert(NBATCH % NS == 0 && QB % RPI == 0, "batches come in groups of NS");
  auto batch_row = [&](int b) { return q0 + (int64_t)b * 4 * QB; };
  u32x4 qs[NS][NL];
  auto load = [&](int b, u32x4 (&q)[NL]) {
    const TileRows tr = tile_rows(batch_row(b < NBATCH ? b : NBATCH - 1), n, QB);
    const uint16_t* qt = Q + tr.first * D;
#pragma unroll
    for (int i = 0; i < NL; ++i) q[i] = ld16_row(qt, i * RPI + prow, tr.last, D, pblk * 8);  // rows >= n are never stored
  };
  // the head's fp32 state -> bf16 operands in LDS
  constexpr int NKV4 = D * D / 1024;
  f32x4 kv4[NKV4];
  float zv;
  head_state<D>(a, bh, tid, kv4, zv);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < NS; ++u) {  // in order, as in kv_state_bf16
    load(u, qs[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < NKV4; ++i) {
    const int e = (tid + 256 * i) * 4, ar = e / D, c = e % D;
    KVt[(c + 0) * LD + ar] = __builtin_bit_cast(uint16_t, (__bf16)kv4[i].x);
    KVt[(c + 1) * LD + ar] = __builtin_bit_cast(uint16_t, (__bf16)kv4[i].y);
    KVt[(c + 2) * LD + ar] = __builtin_bit_cast(uint16_t, (__bf16)kv4[i].z);
    KVt[(c + 3) * LD + ar] = __builtin_bit_cast(uint16_t, (__bf16)kv4[i].w);
  }
  for (int e = tid; e < 16 * D; e += 256) Zr[e / D * LD + e % D] = 0;
  __syncthreads();
  if (tid < D) {
    const __bf16 hi = (__bf16)zv;
    Zr[tid] = __builtin_bit_cast(uint16_t, hi);
    Zr[LD + tid] = __builtin_bit_cast(uint16_t, (__bf16)(zv - (float)hi));
  }
  __syncthreads();

  // A wave's LDS accesses execute in order, so its private tile needs no barrier, and the
  // outputs can overwrite phi(Q) once its operands are read.
  auto compute = [&](int b, const u32x4 (&q)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) st16(&Ts[sofs(i * RPI + prow, pblk)], phi_bf16x8(q[i]));
    u32x4 qf[BB][KS];
#pragma unroll
    for (int bb = 0; bb < BB; ++bb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[bb][ks] = ld16(&Ts[sofs(bb * 16 + l16, 4 * ks + g)]);
    f32x4 acc[BB][NC];
    f32x4 accd[BB];
#pragma unroll
    for (int bb = 0; bb < BB; ++bb) {
      accd[bb] = zero4();
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[bb][c] = zero4();
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const u32x4 kvop = ld16(&KVt[(c * 16 + l16) * LD + ks * 32 + g * 8]);
#pragma unroll
        for (int bb = 0; bb < BB; ++bb) acc[bb][c] = mfma_bf16(kvop, qf[bb][ks], acc[bb][c]);
      }
      const u32x4 zop = ld16(&Zr[l16 * LD + ks * 32 + g * 8]);
#pragma unroll
      for (int bb = 0; bb < BB; ++bb) accd[bb] = mfma_bf16(zop, qf[bb][ks], accd[bb]);
    }
#pragma unroll
    for (int bb = 0; bb < BB; ++bb) {
      const float inv = __builtin_amdgcn_rcpf(__shfl(accd[bb][0] + accd[bb][1], l16));  // den > 0
      // lane (l16, g) holds features 16 c + 4 g + r of query l16: 8 bytes of its output row
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u32x2 o;
        o.x = pack_bf16(acc[bb][c][0] * inv, acc[bb][c][1] * inv);
        o.y = pack_bf16(acc[bb][c][2] * inv, acc[bb][c][3] * inv);
        *reinterpret_cast<u32x2*>(&Ts[sofs(bb * 16 + l16, 2 * c + (g >> 1)) + 4 * (g & 1)]) = o;
      }
    }
    const int64_t r0 = batch_row(b);
    char* ot = reinterpret_cast<char*>(O + r0 * D);  // uniform tile base
    u32x4 v[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) v[i] = ld16(&Ts[sofs(i * RPI + prow, pblk)]);
    // Non-temporal stores: the rows are not read again here, and a store that allocates in the
    // memory-side cache first writes back what an earlier kernel left dirty there (measured in
    // the bench step, after the chunked causal kernel and a decode step: 0.201 -> 0.196 ms)
    if (r0 + QB <= n) {  // uniform: only the last tile of a head can be partial
#pragma unroll
      for (int i = 0; i < NL; ++i) st16_nt(ot + (uint32_t)(((i * RPI + prow) * D + pblk * 8) * 2), v[i]);
    } else {
#pragma unroll
      for (int i = 0; i < NL; ++i)
        if ((int64_t)(i * RPI + prow) < n - r0)  // rows >= n are not stored
          st16_nt(ot + (uint32_t)(((i * RPI + prow) * D + pblk * 8) * 2), v[i]);
    }
  };
  for (int b = 0; b < NBATCH; b += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      compute(b + u, qs[u]);
      __builtin_amdgcn_sched_barrier(0);
      load(b + u + NS, qs[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// fp32 output: the same orientation with each product of fp32 values taken from two-term bf16
// splits (split8, mfma_split in la_common.h).  The workgroup holds its head's KV^T in LDS as two bf16 planes, hi
// and lo (rows = value columns, 16-byte pieces permuted by the row: pswz); a lane loads 32 bytes
// of its query row per 32-feature step, features 32 ks + 8 g .. + 7, the k slots of both
// operands.  The normaliser phi(q).z is a plain fp32 dot product.  A wave takes its queries in
// steps of BB 16-query blocks, which share every KV^T read from LDS, and loads the next step's
// rows while it computes (unconditional loads; rows past the end read row n - 1 and are not
// stored).  The KV^T reads are kept inside the loop (an empty asm statement hides that they
// repeat): hoisted out of it, KV^T would occupy the register file.
template <int D, class TB, int QTV>
__global__ __launch_bounds__(256) void nc_out_f32(NcOutArgs a, TB tb) {
  constexpr int NC = D / 16;
  constexpr int KA = D / 32;                 // 32-feature steps of the reduction
  constexpr int BB = D == 64 ? 2 : 1;        // 16-query blocks per step
  constexpr int64_t QT = QTV;  // queries per workgroup (nc_queries, or less when the heads are few)
  constexpr int QPW = (int)QT / 4;
  constexpr int NB = QPW / (16 * BB);        // steps per wave
  static_assert(NB % 2 == 0, "steps come in pairs");
  __shared__ __attribute__((aligned(16))) uint16_t KvH[D * D];
  __shared__ __attribute__((aligned(16))) uint16_t KvL[D * D];
  __shared__ float zs[D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t tiles = (a.n + QT - 1) / QT;
  const int64_t bh = blockIdx.x / tiles;
  const HeadSpan sp = head_span(tb, a.n, bh);
  if ((blockIdx.x % tiles) * QT >= sp.n) return;  // a tile past a shorter sequence's end
  const int64_t n = sp.n;
  const int64_t q0 = (blockIdx.x % tiles) * QT + wave * QPW;
  constexpr int NKV4 = D * D / 1024;
  f32x4 kv4[NKV4];
  float zv;
  head_state<D>(a, bh, tid, kv4, zv);
#pragma unroll
  for (int i = 0; i < NKV4; ++i) {  // KV[ar][c .. c + 3] -> KV^T rows c .. c + 3, column ar
    const int e = (tid + 256 * i) * 4, ar = e / D, c = e % D;
    u32x2 h, l;
    split4(kv4[i], h, l);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t hw = j < 2 ? h.x : h.y, lw = j < 2 ? l.x : l.y;
      KvH[pswz<D>(c + j, ar)] = (uint16_t)((j & 1) ? hw >> 16 : hw);
      KvL[pswz<D>(c + j, ar)] = (uint16_t)((j & 1) ? lw >> 16 : lw);
    }
  }
  if (tid < D) zs[tid] = zv;
  __syncthreads();

  const float* Q = reinterpret_cast<const float*>(a.q) + sp.row0 * D;
  float* O = reinterpret_cast<float*>(a.out) + sp.row0 * D;
  auto load = [&](int st, f32x4 (&q)[BB][2 * KA]) {
#pragma unroll
    for (int bb = 0; bb < BB; ++bb) {
      const int64_t row = q0 + (int64_t)(BB * st + bb) * 16 + l16;
      const int64_t r = row < n ? row : n - 1;
#pragma unroll
      for (int m = 0; m < 2 * KA; ++m)
        q[bb][m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Q + r * D + (m >> 1) * 32 + g * 8 + (m & 1) * 4));
    }
  };
  auto compute = [&](int st, const f32x4 (&q)[BB][2 * KA]) {
    int l16o = l16;
    asm volatile("" : "+v"(l16o));  // KV^T is re-read every step
    f32x4 acc[BB][NC];
    float dpart[BB];
#pragma unroll
    for (int bb = 0; bb < BB; ++bb) {
      dpart[bb] = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[bb][c] = zero4();
    }
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) {
      u32x4 qh[BB], ql[BB];
#pragma unroll
      for (int bb = 0; bb < BB; ++bb) {
        f32x4 x0 = q[bb][2 * ks], x1 = q[bb][2 * ks + 1];
        x0.x = phi(x0.x);
        x0.y = phi(x0.y);
        x0.z = phi(x0.z);
        x0.w = phi(x0.w);
        x1.x = phi(x1.x);
        x1.y = phi(x1.y);
        x1.z = phi(x1.z);
        x1.w = phi(x1.w);
        const float* zp = zs + ks * 32 + g * 8;
        dpart[bb] += x0.x * zp[0] + x0.y * zp[1] + x0.z * zp[2] + x0.w * zp[3] +
                     x1.x * zp[4] + x1.y * zp[5] + x1.z * zp[6] + x1.w * zp[7];
        split8(x0, x1, qh[bb], ql[bb]);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int o = pswz<D>(c * 16 + l16o, ks * 32 + g * 8);
        const u32x4 kh = ld16(&KvH[o]), kl = ld16(&KvL[o]);
#pragma unroll
        for (int bb = 0; bb < BB; ++bb) {
          acc[bb][c] = mfma_split(kh, kl, qh[bb], ql[bb], acc[bb][c]);
        }
      }
    }
#pragma unroll
    for (int bb = 0; bb < BB; ++bb) {
      const float den = sum_over_groups(dpart[bb]);
      const int64_t row = q0 + (int64_t)(BB * st + bb) * 16 + l16;
      if (row < n) {
        // one IEEE division per row, then products (within 1.5 ulp of a division per element);
        // a denominator too small for its reciprocal to be finite keeps the exact divisions
        const float inv = 1.0f / den;
        const bool tiny = !(den >= 0x1p-120f);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          f32x4 o = {acc[bb][c][0] * inv, acc[bb][c][1] * inv, acc[bb][c][2] * inv, acc[bb][c][3] * inv};
          if (tiny) o = f32x4{acc[bb][c][0] / den, acc[bb][c][1] / den, acc[bb][c][2] / den, acc[bb][c][3] / den};
          *reinterpret_cast<f32x4*>(O + row * D + c * 16 + g * 4) = o;
        }
      }
    }
  };
  f32x4 qa[BB][2 * KA], qb[BB][2 * KA];
  load(0, qa);
  for (int st = 0; st < NB; st += 2) {
    load(st + 1, qb);
    compute(st, qa);
    load(st + 2, qa);  // past the wave's last step: clamped rows, never stored
    compute(st + 1, qb);
  }
}

// ----------------------------------------------------------------------------- launchers
template <int D, class TB>
static void launch_kv_state_tb(const KvStateArgs& a, int dtype, hipStream_t s, const TB& tb) {
  const int64_t blocks = a.groups * a.slices;
  if (dtype == 1 && D == 64)
    hipLaunchKernelGGL((kv_state_bf16_waves<64, TB>), dim3((unsigned)blocks), dim3(256), 0, s, a, tb);
  else if (dtype == 1)
    hipLaunchKernelGGL((kv_state_bf16<D, TB>), dim3((unsigned)blocks), dim3(256), 0, s, a, tb);
  else
    hipLaunchKernelGGL((kv_state_f32<D, TB>), dim3((unsigned)blocks), dim3(256), 0, s, a, tb);
}

template <int D>
static hipError_t launch_kv_state_t(const KvStateArgs& a, int dtype, hipStream_t s, const SeqTable* tab) {
  if (tab)
    launch_kv_state_tb<D>(a, dtype, s, *tab);
  else
    launch_kv_state_tb<D>(a, dtype, s, NoTable{});
  return hipGetLastError();
}

hipError_t launch_kv_state(const KvStateArgs& a, int d, int dtype, hipStream_t s, const SeqTable* tab) {
  return d == 64 ? launch_kv_state_t<64>(a, dtype, s, tab) : launch_kv_state_t<128>(a, dtype, s, tab);
}

template <int D>
static hipError_t launch_state_reduce_t(const KvStateArgs& a, hipStream_t s) {
  constexpr int64_t BPG = ((D * D + D) / 4 + 255) / 256;
  hipLaunchKernelGGL(state_reduce<D>, dim3((unsigned)(a.groups * BPG)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_state_reduce(const KvStateArgs& a, int d, hipStream_t s) {
  return d == 64 ? launch_state_reduce_t<64>(a, s) : launch_state_reduce_t<128>(a, s);
}

// bf16 output tiles: nc_queries(D, 1) queries per workgroup (256 at D = 64); at D = 128 halved,
// down to 2048, while the launch would leave compute units idle (fewer than 256 workgroups, e.g.
// a few heads)
template <int D, class TB, int QTV>
static void launch_nc_out_bf16(const NcOutArgs& a, hipStream_t s, const TB& tb) {
  const int64_t tiles = (a.n + QTV - 1) / QTV;
  if constexpr (QTV > (D == 128 ? 2048 : 512)) {
    if (a.bh * tiles < 256) {
      launch_nc_out_bf16<D, TB, QTV / 2>(a, s, tb);
      return;
    }
  }
  hipLaunchKernelGGL((nc_out_bf16<D, TB, QTV>), dim3((unsigned)(a.bh * tiles)), dim3(256), 0, s, a, tb);
}

// fp32 output tiles likewise, down to 256 queries at D = 64 and 128 at D = 128 (the smallest
// tiles that keep the kernel's steps in pairs)
template <int D, class TB, int QTV>
static void launch_nc_out_f32(const NcOutArgs& a, hipStream_t s, const TB& tb) {
  const int64_t tiles = (a.n + QTV - 1) / QTV;
  if constexpr (QTV > (D == 64 ? 256 : 128)) {
    if (a.bh * tiles < 256) {
      launch_nc_out_f32<D, TB, QTV / 2>(a, s, tb);
      return;
    }
  }
  hipLaunchKernelGGL((nc_out_f32<D, TB, QTV>), dim3((unsigned)(a.bh * tiles)), dim3(256), 0, s, a, tb);
}

template <int D, class TB>
static void launch_nc_out_tb(const NcOutArgs& a, int dtype, hipStream_t s, const TB& tb) {
  if (dtype == 1)
    launch_nc_out_bf16<D, TB, (int)nc_queries(D, 1)>(a, s, tb);
  else
    launch_nc_out_f32<D, TB, (int)nc_queries(D, 0)>(a, s, tb);
}

template <int D>
static hipError_t launch_nc_out_t(const NcOutArgs& a, int dtype, hipStream_t s, const SeqTable* tab) {
  if (tab)
    launch_nc_out_tb<D>(a, dtype, s, *tab);
  else
    launch_nc_out_tb<D>(a, dtype, s, NoTable{});
  return hipGetLastError();
}

hipError_t launch_nc_out(const NcOutArgs& a, int d, int dtype, hipStream_t s, const SeqTable* tab) {
  return d == 64 ? launch_nc_out_t<64>(a, dtype, s, tab) : launch_nc_out_t<128>(a, dtype, s, tab);
}

}  // namespace la
