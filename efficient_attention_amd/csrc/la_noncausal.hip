// la_noncausal.hip -- non-causal linear attention on gfx950, and the per-block state sums that
// the causal path reuses.
//
// Math ("Efficient Transformers: Linear Attention and Flash Attention", section "Linear
// attention: reordering the matmuls, not shrinking them", eq. Attention_i):
//     KV = sum_j phi(k_j) v_j^T  (D x d),  z = sum_j phi(k_j)  (D),
//     out_i = phi(q_i) KV / phi(q_i) z.
// Because the sums split over any partition of the keys (associativity, section "Worked
// example"), stage 1 sums slices of keys in parallel and the last workgroup of each group
// adds the slices in a fixed order (deterministic, no float atomics); stage 2 streams the
// queries.
//
// Kernels
//   kv_state_*   stage 1.  Grid = groups x slices (1-D).  A group is a contiguous token range
//                of one head; its result, [KV (D x D) | z (D)] fp32, lands in `state[group]`.
//   nc_out_*     stage 2.  Grid = heads x query tiles (1-D).
#include "la_common.h"
#include "la_kernels.h"

namespace la {

// ----------------------------------------------------------------------------- stage 1
// Group bookkeeping shared by the bf16 and fp32 variants.
struct GroupRange {
  int64_t g, bh, s;   // group, head, slice
  int64_t t0, t1;     // token range [t0, t1) of this slice within the head
};

__device__ __forceinline__ GroupRange group_range(const KvStateArgs& a) {
  GroupRange r;
  r.g = blockIdx.x / a.slices;
  r.s = blockIdx.x % a.slices;
  r.bh = r.g / a.groups_per_head;
  int64_t seg = r.g % a.groups_per_head;
  int64_t gs = seg * a.group_len;
  int64_t ge = gs + a.group_len < a.n ? gs + a.group_len : a.n;
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

// bf16 stage 1.  Tile = T tokens with T*D = 16384, so each of the 256 threads owns one 8x8
// block of K and one of V per tile.  A block is loaded as 8 rows of 16 bytes, phi is applied
// to K in fp32 and rounded to bf16, and both blocks are transposed in registers so LDS holds
// token-contiguous rows: Kt[a][t] = phi(K)[t][a], Vt[c][t] = V[t][c].  That is the layout the
// MFMA wants, because the reduction index of phi(K)^T V is the token.
template <int D>
__global__ __launch_bounds__(256) void kv_state_bf16(KvStateArgs a) {
  constexpr int T = 16384 / D;       // tokens per tile
  constexpr int TS = tsize<D, T>();  // token-major tile (see tofs)
  constexpr int FB = D / 8;          // feature blocks per token row
  constexpr int NA = D / 64;         // a-tiles (of 16 rows) per wave
  constexpr int NC = D / 16;         // c-tiles
  // one buffer: the two token-major tiles, later reused for the fp32 result [KV | z]
  static_assert(2 * TS * 2 >= (D * D + D) * 4, "result must fit in the tile buffers");
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * TS];
  uint16_t* Kt = lds;
  uint16_t* Vt = lds + TS;

  const GroupRange gr = group_range(a);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int tb = tid / FB, fb = tid % FB;  // this thread's 8x8 block in the tile
  const uint16_t* K = reinterpret_cast<const uint16_t*>(a.k) + gr.bh * a.n * D;
  const uint16_t* V = reinterpret_cast<const uint16_t*>(a.v) + gr.bh * a.n * D;

  f32x4 acc[NA][NC];
  float zacc[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    zacc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[i][c] = zero4();
  }

  u32x4 kr[8], vr[8];
  auto load_tile = [&](int64_t t0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      kr[r] = ld16_clamp(K, t0 + tb * 8 + r, gr.t1, D, fb * 8);
      vr[r] = ld16_clamp(V, t0 + tb * 8 + r, gr.t1, D, fb * 8);
    }
  };

  if (gr.t0 < gr.t1) load_tile(gr.t0);
  for (int64_t t0 = gr.t0; t0 < gr.t1; t0 += T) {
    // phi on K (invalid rows forced to zero after phi), transpose, write LDS
    u32x4 tk[8], tv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      bool ok = t0 + tb * 8 + r < gr.t1;
      kr[r] = ok ? phi_bf16x8(kr[r]) : zero_u4();
      vr[r] = ok ? vr[r] : zero_u4();
    }
    transpose8x8(kr, tk);
    transpose8x8(vr, tv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      st16(&Kt[tofs<T>(fb * 8 + e, tb * 8)], tk[e]);
      st16(&Vt[tofs<T>(fb * 8 + e, tb * 8)], tv[e]);
    }
    if (t0 + T < gr.t1) load_tile(t0 + T);  // in flight through the MFMA phase
    __syncthreads();
#pragma unroll
    for (int s = 0; s < T / 32; ++s) {
      u32x4 bv[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) bv[c] = ld16(&Vt[tofs<T>(c * 16 + l16, s * 32 + g * 8)]);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int at = wave * NA + i;
        u32x4 ak = ld16(&Kt[tofs<T>(at * 16 + l16, s * 32 + g * 8)]);
        zacc[i] += sum_bf16x8(ak);
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[i][c] = mfma_bf16(ak, bv[c], acc[i][c]);
      }
    }
    __syncthreads();
  }

  // results -> LDS (fp32, reusing the tile buffers) -> global
  float* kv_lds = reinterpret_cast<float*>(lds);
  float* z_lds = kv_lds + D * D;
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int at = wave * NA + i;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) kv_lds[(at * 16 + g * 4 + r) * D + c * 16 + l16] = acc[i][c][r];
    float zs = sum_over_groups(zacc[i]);
    if (g == 0) z_lds[at * 16 + l16] = zs;
  }
  __syncthreads();
  publish_state<D>(a, gr, kv_lds);
}

// fp32 stage 1: tile of 64 tokens kept in natural layout (the fp32 MFMA takes one k value
// per lane, so no transpose is needed).
template <int D>
__global__ __launch_bounds__(256) void kv_state_f32(KvStateArgs a) {
  constexpr int T = 64;
  constexpr int LD = D + 4;
  constexpr int NA = D / 64;
  constexpr int NC = D / 16;
  __shared__ __attribute__((aligned(16))) float Kn[T * LD];
  __shared__ __attribute__((aligned(16))) float Vn[T * LD];
  __shared__ __attribute__((aligned(16))) float kv_lds[D * D + D];  // [KV | z]
  float* z_lds = kv_lds + D * D;

  const GroupRange gr = group_range(a);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const float* K = reinterpret_cast<const float*>(a.k) + gr.bh * a.n * D;
  const float* V = reinterpret_cast<const float*>(a.v) + gr.bh * a.n * D;

  f32x4 acc[NA][NC];
  float zacc[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    zacc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[i][c] = zero4();
  }
  for (int64_t t0 = gr.t0; t0 < gr.t1; t0 += T) {
    for (int idx = tid; idx < T * (D / 4); idx += 256) {
      int row = idx / (D / 4), c4 = idx % (D / 4);
      int64_t tok = t0 + row;
      f32x4 kk = zero4(), vv = zero4();
      if (tok < gr.t1) {
        kk = *reinterpret_cast<const f32x4*>(K + tok * D + c4 * 4);
        vv = *reinterpret_cast<const f32x4*>(V + tok * D + c4 * 4);
        kk.x = phi(kk.x);
        kk.y = phi(kk.y);
        kk.z = phi(kk.z);
        kk.w = phi(kk.w);
      }
      *reinterpret_cast<f32x4*>(&Kn[row * LD + c4 * 4]) = kk;
      *reinterpret_cast<f32x4*>(&Vn[row * LD + c4 * 4]) = vv;
    }
    __syncthreads();
#pragma unroll 4
    for (int s = 0; s < T / 4; ++s) {
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int at = wave * NA + i;
        float ak = Kn[(s * 4 + g) * LD + at * 16 + l16];
        zacc[i] += ak;
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[i][c] = mfma_f32(ak, Vn[(s * 4 + g) * LD + c * 16 + l16], acc[i][c]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int at = wave * NA + i;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) kv_lds[(at * 16 + g * 4 + r) * D + c * 16 + l16] = acc[i][c][r];
    float zs = sum_over_groups(zacc[i]);
    if (g == 0) z_lds[at * 16 + l16] = zs;
  }
  __syncthreads();
  publish_state<D>(a, gr, kv_lds);
}

// ----------------------------------------------------------------------------- stage 2
// bf16 output.  The workgroup turns its head's fp32 [KV | z] into bf16 MFMA operands in LDS:
// KVt[c][a] = KV[a][c], and a 16-row "normaliser" tile whose rows 0 and 1 hold z split into a
// bf16 high part and a bf16 residual (so phi(q).z keeps ~16 significant bits).  Each wave then
// takes 16 queries at a time and computes out^T = [KV^T ; z] phi(Q)^T with queries as the MFMA
// column index: a lane's 16-byte load of a query row is directly its operand.
template <int D>
__global__ __launch_bounds__(256) void nc_out_bf16(NcOutArgs a) {
  constexpr int LD = D + 16;  // row stride of 8 mod 64 dwords: conflict-free 16-row reads
  constexpr int NC = D / 16;
  constexpr int KS = D / 32;
  constexpr int QPW = kNcQueries / 4;  // queries per wave
  __shared__ __attribute__((aligned(16))) uint16_t KVt[D * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Zr[16 * LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t tiles = (a.n + kNcQueries - 1) / kNcQueries;
  const int64_t bh = blockIdx.x / tiles;
  const int64_t q0 = (blockIdx.x % tiles) * kNcQueries + wave * QPW;
  const float* st = a.state + bh * (D * D + D);

  // the head's fp32 state: every load issued before any is used (one memory latency)
  constexpr int NKV4 = D * D / 4 / 256;
  f32x4 kv4[NKV4];
#pragma unroll
  for (int i = 0; i < NKV4; ++i) kv4[i] = reinterpret_cast<const f32x4*>(st)[tid + 256 * i];
  const float zv = tid < D ? st[D * D + tid] : 0.f;
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

  const uint16_t* Q = reinterpret_cast<const uint16_t*>(a.q) + bh * a.n * D;
  uint16_t* O = reinterpret_cast<uint16_t*>(a.out) + bh * a.n * D;

  // query blocks of 16 rows go in batches of BB, the next batch in flight during compute
  constexpr int BB = D == 64 ? 4 : 2;
  constexpr int NBATCH = QPW / 16 / BB;
  u32x4 qr[BB][KS];
  auto load_batch = [&](int64_t r0) {
#pragma unroll
    for (int b = 0; b < BB; ++b)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qr[b][ks] = ld16_clamp(Q, r0 + b * 16 + l16, a.n, D, ks * 32 + g * 8);  // rows >= n are never stored
  };
  load_batch(q0);
  for (int bt = 0; bt < NBATCH; ++bt) {
    u32x4 qf[BB][KS];
#pragma unroll
    for (int b = 0; b < BB; ++b)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[b][ks] = phi_bf16x8(qr[b][ks]);
    if (bt + 1 < NBATCH) load_batch(q0 + (bt + 1) * 16 * BB);
#pragma unroll
    for (int b = 0; b < BB; ++b) {
      const int64_t row = q0 + (bt * BB + b) * 16 + l16;
      f32x4 acc[NC];
      f32x4 accd = zero4();
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
          acc[c] = mfma_bf16(ld16(&KVt[(c * 16 + l16) * LD + ks * 32 + g * 8]), qf[b][ks], acc[c]);
        accd = mfma_bf16(ld16(&Zr[l16 * LD + ks * 32 + g * 8]), qf[b][ks], accd);
      }
      const float den = __shfl(accd[0] + accd[1], l16);
      const float inv = 1.0f / den;
      if (row < a.n) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          u32x2 o;
          o.x = pack_bf16(acc[c][0] * inv, acc[c][1] * inv);
          o.y = pack_bf16(acc[c][2] * inv, acc[c][3] * inv);
          *reinterpret_cast<u32x2*>(O + row * D + c * 16 + g * 4) = o;
        }
      }
    }
  }
}

// fp32 output: same orientation with the fp32 MFMA (one k value per lane).  A lane loads 16
// bytes of its query row, a[16m + 4g .. +3]; k-step 4m+e uses a = 16m + 4g + e on both
// operands.  The normaliser phi(q).z is a plain fp32 dot product.
template <int D>
__global__ __launch_bounds__(256) void nc_out_f32(NcOutArgs a) {
  constexpr int LD = D + 4;
  constexpr int NC = D / 16;
  constexpr int QPW = kNcQueries / 4;
  __shared__ __attribute__((aligned(16))) float KVt[D * LD];
  __shared__ float zs[D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t tiles = (a.n + kNcQueries - 1) / kNcQueries;
  const int64_t bh = blockIdx.x / tiles;
  const int64_t q0 = (blockIdx.x % tiles) * kNcQueries + wave * QPW;
  const float* st = a.state + bh * (D * D + D);
  constexpr int NKV4 = D * D / 4 / 256;
  f32x4 kv4[NKV4];
#pragma unroll
  for (int i = 0; i < NKV4; ++i) kv4[i] = reinterpret_cast<const f32x4*>(st)[tid + 256 * i];
#pragma unroll
  for (int i = 0; i < NKV4; ++i) {
    const int e = (tid + 256 * i) * 4, ar = e / D, c = e % D;
    KVt[(c + 0) * LD + ar] = kv4[i].x;
    KVt[(c + 1) * LD + ar] = kv4[i].y;
    KVt[(c + 2) * LD + ar] = kv4[i].z;
    KVt[(c + 3) * LD + ar] = kv4[i].w;
  }
  if (tid < D) zs[tid] = st[D * D + tid];
  __syncthreads();

  const float* Q = reinterpret_cast<const float*>(a.q) + bh * a.n * D;
  float* O = reinterpret_cast<float*>(a.out) + bh * a.n * D;
  for (int blk = 0; blk < QPW / 16; ++blk) {
    const int64_t row = q0 + blk * 16 + l16;
    f32x4 acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = zero4();
    float dpart = 0.f;
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
      f32x4 qv = row < a.n ? *reinterpret_cast<const f32x4*>(Q + row * D + m * 16 + g * 4) : zero4();
      float qf[4] = {phi(qv.x), phi(qv.y), phi(qv.z), phi(qv.w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) dpart += qf[e] * zs[m * 16 + g * 4 + e];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        f32x4 kv = *reinterpret_cast<const f32x4*>(&KVt[(c * 16 + l16) * LD + m * 16 + g * 4]);
        acc[c] = mfma_f32(kv.x, qf[0], acc[c]);
        acc[c] = mfma_f32(kv.y, qf[1], acc[c]);
        acc[c] = mfma_f32(kv.z, qf[2], acc[c]);
        acc[c] = mfma_f32(kv.w, qf[3], acc[c]);
      }
    }
    float den = sum_over_groups(dpart);
    if (row < a.n) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        f32x4 o = {acc[c][0] / den, acc[c][1] / den, acc[c][2] / den, acc[c][3] / den};
        *reinterpret_cast<f32x4*>(O + row * D + c * 16 + g * 4) = o;
      }
    }
  }
}

// ----------------------------------------------------------------------------- launchers
template <int D>
static hipError_t launch_kv_state_t(const KvStateArgs& a, int dtype, hipStream_t s) {
  const int64_t blocks = a.groups * a.slices;
  if (dtype == 1)
    hipLaunchKernelGGL(kv_state_bf16<D>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(kv_state_f32<D>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_kv_state(const KvStateArgs& a, int d, int dtype, hipStream_t s) {
  return d == 64 ? launch_kv_state_t<64>(a, dtype, s) : launch_kv_state_t<128>(a, dtype, s);
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

template <int D>
static hipError_t launch_nc_out_t(const NcOutArgs& a, int dtype, hipStream_t s) {
  const int64_t blocks = a.bh * ((a.n + kNcQueries - 1) / kNcQueries);
  if (dtype == 1)
    hipLaunchKernelGGL(nc_out_bf16<D>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(nc_out_f32<D>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_nc_out(const NcOutArgs& a, int d, int dtype, hipStream_t s) {
  return d == 64 ? launch_nc_out_t<64>(a, dtype, s) : launch_nc_out_t<128>(a, dtype, s);
}

}  // namespace la
