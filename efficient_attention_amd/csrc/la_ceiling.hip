// la_ceiling.hip -- memory-system measurements that bound the linear-attention kernels
// (include/la_ceiling.h).  A memory-bound kernel's time is at least its bytes over the bandwidth
// the memory system gives its access pattern (Hoefler, "Let's Stop Calling Everything 'Linear
// Attention'", section 2: t_mem >= T_mem / B_effective); these kernels measure B_effective for a
// plain copy, a read-only stream and the chunked causal kernel's own pattern, each computing a
// checkable result.
#include <limits.h>
#include <stdint.h>

#include "la_ceiling.h"
#include "la_common.h"
#include "linattn.h"

namespace la {
namespace {

constexpr int kReadUnroll = 4;
constexpr int kStreamBlocks = 2048;

// dst = src: one 16-byte piece per thread, 4 KB per workgroup, one workgroup per 4 KB of the
// buffer, non-temporal both ways.  Of the copy variants measured on this device this is the
// fastest (6.4 TB/s over 2 GiB): the workgroups are short and start in address order, so the
// rows written at any moment lie close together.  Long-lived workgroups that stride over the
// buffer, or that each stream their own range, copy at 5.0-5.5 TB/s.
__global__ __launch_bounds__(256) void ceiling_copy(const u32x4* src, u32x4* dst, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Every 16-byte piece read once; workgroup w streams the w-th of gridDim.x contiguous ranges
// (four pieces per thread and step, non-temporal loads: 6.9-7.0 TB/s over 2 GiB on this device,
// against 6.3-6.4 with cached loads) and writes the XOR of its words to sink[w].
__global__ __launch_bounds__(256) void ceiling_read(const u32x4* src, int64_t n16, uint32_t* sink) {
  __shared__ uint32_t part[4];
  uint32_t acc = 0;
  const int64_t len = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * len;
  const int64_t b1 = b0 + len < n16 ? b0 + len : n16;
  for (int64_t i0 = b0 + threadIdx.x; i0 < b1; i0 += 256 * kReadUnroll) {
    u32x4 r[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t i = i0 + u * 256;
      r[u] = i < b1 ? __builtin_nontemporal_load(src + i) : zero_u4();
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// The chunked causal kernel's memory pattern (causal_bf16 at D = 128, C = 128) with out = q + k + v.
// K and V of a chunk pass through LDS as whole rows (V double-buffered, like the real kernel);
// the next chunk's K, V and query rows are loaded in three groups spread over the chunk; each wave
// owns query tile it (tiles s and 7 - s share a SIMD) and stores its 16 output rows in 64-byte
// pieces.  104 KB of LDS: one workgroup per compute unit, as the real kernel (141 KB).
constexpr int kPD = 128, kPC = 128, kPLD = kPD + 8;
__global__ __launch_bounds__(512) void ceiling_causal_pattern(const uint16_t* q, const uint16_t* k,
                                                              const uint16_t* v, uint16_t* out, int64_t n,
                                                              int64_t segs, int64_t seg_len) {
  constexpr int NT = 512, PPR = kPD / 8, RPK = kPC * PPR / NT, KA = kPD / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kPC * kPLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2 * kPC * kPLD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t bh = blockIdx.x / segs, seg = blockIdx.x % segs;
  const int64_t t0 = seg * seg_len;
  if (t0 >= n) return;
  const int64_t t1 = t0 + seg_len < n ? t0 + seg_len : n;
  const uint16_t* Q = q + bh * n * kPD;
  const uint16_t* K = k + bh * n * kPD;
  const uint16_t* V = v + bh * n * kPD;
  uint16_t* O = out + bh * n * kPD;
  const int it = wave < 4 ? wave : 11 - wave;
  auto prow = [&](int p) { return tid / PPR + p * (NT / PPR); };
  const int pcol = (tid % PPR) * 8;
  u32x4 kr[RPK], vr[RPK], qr[KA], qc[KA];
  auto load_k = [&](int64_t c0) {
#pragma unroll
    for (int p = 0; p < RPK; ++p) kr[p] = ld16_clamp_nt(K, c0 + prow(p), t1, kPD, pcol);
  };
  auto load_v = [&](int64_t c0) {
#pragma unroll
    for (int p = 0; p < RPK; ++p) vr[p] = ld16_clamp_nt(V, c0 + prow(p), t1, kPD, pcol);
  };
  auto load_q = [&](int64_t c0) {
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) qr[ks] = ld16_clamp_nt(Q, c0 + it * 16 + l16, t1, kPD, ks * 32 + g * 8);
  };
  auto store_k = [&]() {
#pragma unroll
    for (int p = 0; p < RPK; ++p) st16(&Ks[prow(p) * kPLD + pcol], kr[p]);
  };
  auto store_v = [&](uint16_t* Vt) {
#pragma unroll
    for (int p = 0; p < RPK; ++p) st16(&Vt[prow(p) * kPLD + pcol], vr[p]);
  };
  // out rows of this wave's tile, columns ks * 32 + 8 g .. + 7: (q + k) + v in fp32, rounded
  auto emit = [&](int64_t c0, const uint16_t* Vt, int ks) {
    const int r = it * 16 + l16, col = ks * 32 + g * 8;
    const u32x4 kk = ld16(&Ks[r * kPLD + col]);
    const u32x4 vv = ld16(&Vt[r * kPLD + col]);
    const u32x4 a = qc[ks];
    u32x4 o;
    o.x = pack_bf16(bf_lo(a.x) + bf_lo(kk.x) + bf_lo(vv.x), bf_hi(a.x) + bf_hi(kk.x) + bf_hi(vv.x));
    o.y = pack_bf16(bf_lo(a.y) + bf_lo(kk.y) + bf_lo(vv.y), bf_hi(a.y) + bf_hi(kk.y) + bf_hi(vv.y));
    o.z = pack_bf16(bf_lo(a.z) + bf_lo(kk.z) + bf_lo(vv.z), bf_hi(a.z) + bf_hi(kk.z) + bf_hi(vv.z));
    o.w = pack_bf16(bf_lo(a.w) + bf_lo(kk.w) + bf_lo(vv.w), bf_hi(a.w) + bf_hi(kk.w) + bf_hi(vv.w));
    const int64_t row = c0 + r;
    if (row < t1) st16(O + row * kPD + col, o);
  };
  load_k(t0);
  load_v(t0);
  load_q(t0);
  store_k();
  store_v(Vs);
  int buf = 0;
  for (int64_t c0 = t0; c0 < t1; c0 += kPC, buf ^= 1) {
    __syncthreads();  // this chunk's K and V in LDS
    const uint16_t* Vc = Vs + buf * (kPC * kPLD);
#pragma unroll
    for (int ks = 0; ks < KA; ++ks) qc[ks] = qr[ks];
    __builtin_amdgcn_sched_barrier(0);
    load_k(c0 + kPC);
    __builtin_amdgcn_sched_barrier(0);
    emit(c0, Vc, 0);
    emit(c0, Vc, 1);
    __builtin_amdgcn_sched_barrier(0);
    load_v(c0 + kPC);
    __builtin_amdgcn_sched_barrier(0);
    emit(c0, Vc, 2);
    emit(c0, Vc, 3);
    __builtin_amdgcn_sched_barrier(0);
    load_q(c0 + kPC);
    __builtin_amdgcn_sched_barrier(0);
    store_v(Vs + (buf ^ 1) * (kPC * kPLD));
    __syncthreads();  // every wave is done reading this chunk's K
    store_k();
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace
}  // namespace la

extern "C" {

size_t la_ceiling_read_sink_words(void) { return (size_t)la::kStreamBlocks; }

int la_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes % 16 != 0) return LA_ERR_SHAPE;
  if (bytes == 0) return LA_OK;
  if (!src || !dst) return LA_ERR_NULL;
  if (!la::aligned16(src) || !la::aligned16(dst)) return LA_ERR_ALIGN;
  if (la::overlaps(src, bytes, dst, bytes)) return LA_ERR_ALIAS;
  const int64_t n16 = (int64_t)(bytes / 16), blocks = (n16 + 255) / 256;
  if (blocks > (int64_t)INT_MAX) return LA_ERR_SHAPE;
  hipLaunchKernelGGL(la::ceiling_copy, dim3((unsigned)blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const la::u32x4*>(src), reinterpret_cast<la::u32x4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

int la_ceiling_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes % 16 != 0) return LA_ERR_SHAPE;
  if (bytes == 0) return LA_OK;
  if (!src || !sink) return LA_ERR_NULL;
  if (!la::aligned16(src) || !la::aligned16(sink)) return LA_ERR_ALIGN;
  if (la::overlaps(src, bytes, sink, la::kStreamBlocks * sizeof(uint32_t))) return LA_ERR_ALIAS;
  hipLaunchKernelGGL(la::ceiling_read, dim3(la::kStreamBlocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const la::u32x4*>(src), (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

int la_ceiling_causal_pattern(const void* q, const void* k, const void* v, void* out, int64_t B,
                              int64_t H, int64_t n, int64_t d, int64_t seg_len, void* stream) {
  if (B < 0 || H < 0 || n < 0) return LA_ERR_SHAPE;
  if (d != la::kPD) return LA_ERR_UNSUPPORTED;
  if (seg_len <= 0 || seg_len % la::kPC != 0) return LA_ERR_SHAPE;
  int64_t bh = 0, e = 0;
  if (__builtin_mul_overflow(B, H, &bh) || __builtin_mul_overflow(bh, n, &e) ||
      __builtin_mul_overflow(e, d * 2, &e))
    return LA_ERR_SHAPE;
  if (bh == 0 || n == 0) return LA_OK;
  if (!q || !k || !v || !out) return LA_ERR_NULL;
  if (!la::aligned16(q) || !la::aligned16(k) || !la::aligned16(v) || !la::aligned16(out)) return LA_ERR_ALIGN;
  const size_t bytes = (size_t)e;
  if (la::overlaps(out, bytes, q, bytes) || la::overlaps(out, bytes, k, bytes) || la::overlaps(out, bytes, v, bytes))
    return LA_ERR_ALIAS;
  const int64_t segs = (n + seg_len - 1) / seg_len;
  if (bh > INT32_MAX / segs) return LA_ERR_SHAPE;
  hipLaunchKernelGGL(la::ceiling_causal_pattern, dim3((unsigned)(bh * segs)), dim3(512), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint16_t*>(q),
                     reinterpret_cast<const uint16_t*>(k), reinterpret_cast<const uint16_t*>(v),
                     reinterpret_cast<uint16_t*>(out), n, segs, seg_len);
  return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // extern "C"
