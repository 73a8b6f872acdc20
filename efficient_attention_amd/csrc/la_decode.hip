// la_decode.hip -- one recurrent decode step of linear attention for many heads, in place.
//
// Per head ("Efficient Transformers: Linear Attention and Flash Attention", section "The
// recurrent view: attention as an RNN"; the state is the fixed-size summary of Active recall
// A5):
//     S <- S + phi(k) v^T,   z <- z + phi(k),   out = phi(q)^T S / phi(q)^T z.
// The step is a pure read-modify-write stream over S (D*D fp32), so there is no MFMA: each of
// the 256 threads owns 4 adjacent columns and D/RG rows, issues all its 16-byte state loads at
// once (non-temporal), updates them with one FMA per element, writes them back (non-temporal) and keeps
// a running column sum of phi(q)_a * S'[a][c].  Partial column sums and the denominator are
// combined through LDS in a fixed order, so the step is bitwise reproducible.
#include "la_common.h"
#include "la_kernels.h"

namespace la {

template <typename T>
__device__ __forceinline__ float load_elem(const void* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const void* p, int64_t i) {
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
}
template <>
__device__ __forceinline__ float load_elem<float>(const void* p, int64_t i) {
  return reinterpret_cast<const float*>(p)[i];
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_step_kernel(DecodeArgs a) {
  constexpr int CG = D / 4;        // column groups of 4
  constexpr int RG = 256 / CG;     // row groups
  constexpr int RPT = D / RG;      // rows per thread
  __shared__ float fq[D], fk[D], vv[D];
  __shared__ float red[RG][D];
  __shared__ float dwave[4];

  const int64_t h = blockIdx.x;
  if (a.active && !a.active[h / a.heads]) return;  // an inactive sequence: state and out untouched
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  float* S = a.S + h * D * D;

  // state loads first: they are independent of everything else.  Non-temporal: the state is read
  // once per step, and allocating it in the memory-side cache would first write back whatever
  // the previous kernel left dirty there (measured: one decode step after the chunked causal
  // forward 0.235 -> 0.200 ms, the whole bench step 2.49 -> 2.44 ms)
  f32x4 s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m)
    s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (int64_t)(rg + RG * m) * D + cg * 4));

  float znew = 0.f, dpart = 0.f;
  if (tid < D) {
    float qv = phi(load_elem<T>(a.q, h * D + tid));
    float kv = phi(load_elem<T>(a.k, h * D + tid));
    fq[tid] = qv;
    fk[tid] = kv;
    vv[tid] = load_elem<T>(a.v, h * D + tid);
    znew = a.z[h * D + tid] + kv;
    a.z[h * D + tid] = znew;
    dpart = qv * znew;
  }
  // denominator: wave sums in lane order, then the (at most 2) waves in order
  if (tid < D) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dpart += __shfl_xor(dpart, off);
    if ((tid & 63) == 0) dwave[tid >> 6] = dpart;
  }
  __syncthreads();

  const f32x4 v4 = *reinterpret_cast<const f32x4*>(&vv[cg * 4]);
  f32x4 num = zero4();
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int row = rg + RG * m;
    const float ka = fk[row], qa = fq[row];
    s[m].x += ka * v4.x;
    s[m].y += ka * v4.y;
    s[m].z += ka * v4.z;
    s[m].w += ka * v4.w;
    // non-temporal: the state is not read again before the next step, and by then the 256 MB
    // memory-side cache has turned over (8192 heads are 541 MB); a normal store would leave up to
    // 256 MB of dirty lines for the next kernel to write back
    __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4*>(S + (int64_t)row * D + cg * 4));
    num.x += qa * s[m].x;
    num.y += qa * s[m].y;
    num.z += qa * s[m].z;
    num.w += qa * s[m].w;
  }
  *reinterpret_cast<f32x4*>(&red[rg][cg * 4]) = num;
  __syncthreads();
  if (tid < D) {
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) acc += red[r][tid];
    float den = dwave[0];
#pragma unroll
    for (int w = 1; w < (D + 63) / 64; ++w) den += dwave[w];
    float o = acc / den;
    if constexpr (sizeof(T) == 2)
      reinterpret_cast<__bf16*>(a.out)[h * D + tid] = (__bf16)o;
    else
      reinterpret_cast<float*>(a.out)[h * D + tid] = o;
  }
}

template <int D>
static hipError_t launch_decode_t(const DecodeArgs& a, int dtype, hipStream_t s) {
  if (dtype == 1)
    hipLaunchKernelGGL((decode_step_kernel<uint16_t, D>), dim3((unsigned)a.bh), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_step_kernel<float, D>), dim3((unsigned)a.bh), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int d, int dtype, hipStream_t s) {
  return d == 64 ? launch_decode_t<64>(a, dtype, s) : launch_decode_t<128>(a, dtype, s);
}

}  // namespace la
