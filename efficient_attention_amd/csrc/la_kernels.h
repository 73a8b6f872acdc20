// la_kernels.h -- argument blocks and launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

// The heads of a batch.  Fixed length (NoTable): head bh is rows [bh * n, (bh + 1) * n) of the
// [B][H][n][d] tensors.  Variable length (SeqTable): each sequence s is the fixed layout's
// [H][n_s][d] block, the blocks packed back to back; with the offsets cu (cu[0] = 0,
// n_s = cu[s + 1] - cu[s]) head bh = s * H + h starts at row H * cu[s] + h * n_s.  The table
// travels by value in the kernel arguments (validated on the host), so it needs no device memory.
constexpr int kMaxSeqs = 256;
struct NoTable {};
struct SeqTable {
  int64_t heads;               // H
  int64_t cu[kMaxSeqs + 1];    // sequence offsets in tokens
};
struct HeadSpan {
  int64_t row0;  // first row of the head
  int64_t n;     // its tokens
};
__device__ __forceinline__ HeadSpan head_span(const NoTable&, int64_t n, int64_t bh) { return {bh * n, n}; }
__device__ __forceinline__ HeadSpan head_span(const SeqTable& t, int64_t, int64_t bh) {
  const int64_t s = bh / t.heads, h = bh % t.heads;
  const int64_t c0 = t.cu[s], ns = t.cu[s + 1] - c0;
  return {t.heads * c0 + h * ns, ns};
}

// Stage-1 state sums over token ranges ("groups": one per head for the non-causal form, one
// per head and leading segment for the causal form), split into `slices` workgroups each.
struct KvStateArgs {
  const void* k;
  const void* v;
  float* partials;      // [groups][slices][D*D + D] fp32 (unused when slices == 1)
  float* state;         // [groups][D*D + D] fp32: KV row-major, then z
  int64_t n;            // tokens per head
  int64_t group_len;    // tokens per group (the last group of a head may be shorter)
  int64_t groups_per_head;
  int64_t groups;       // total groups
  int64_t slices;       // workgroups per group
  int64_t slice_len;    // tokens per workgroup (multiple of the kernel's tile)
};

struct NcOutArgs {
  const void* q;
  void* out;
  const float* state;   // [bh][slices][D*D + D]: a head's state is the sum of its slices
  int64_t slices;
  int64_t n;
  int64_t bh;
};

struct CausalArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const float* seg_state;  // [bh][segs-1][seg_parts][D*D + D]: the leading segments' sums,
                           // each split into seg_parts partials that add up to it (or null)
  int64_t seg_parts;
  const float* s0;         // [bh][D][D] state before token 0 and its key sums z0 [bh][D]
  const float* z0;         //   (both null: zero state)
  float* sn;               // [bh][D][D] and [bh][D]: receive the state after token n-1
  float* zn;               //   (both null: not written)
  int64_t n;
  int64_t bh;
  int64_t segs;            // segments per head
  int64_t seg_len;         // tokens per segment (multiple of chunk)
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  float* S;
  float* z;
  void* out;
  const uint8_t* active;   // [B] device flags: sequences with 0 are skipped (null: all active)
  int64_t heads;           // H (to find a head's sequence)
  int64_t bh;
};

// `tab` null: fixed-length batch (n = a.n for every head); else a variable-length batch whose
// heads are described by *tab, and a.n is the longest sequence (the grids are planned for it;
// workgroups beyond a shorter sequence exit at once).
hipError_t launch_kv_state(const KvStateArgs& a, int d, int dtype, hipStream_t s, const SeqTable* tab = nullptr);
hipError_t launch_state_reduce(const KvStateArgs& a, int d, hipStream_t s);
hipError_t launch_nc_out(const NcOutArgs& a, int d, int dtype, hipStream_t s, const SeqTable* tab = nullptr);
hipError_t launch_causal(const CausalArgs& a, int d, int chunk, int dtype, hipStream_t s, const SeqTable* tab = nullptr);
hipError_t launch_decode(const DecodeArgs& a, int d, int dtype, hipStream_t s);
// sn, zn = s0, z0 (zeros where s0, z0 are null) for every head: the final state of an empty sequence.
hipError_t launch_state_copy(const CausalArgs& a, int d, hipStream_t s);

// ---- FAVOR+ feature map (positive random features; la_favor.hip, la_favor_causal.hip)
// phi(x) = exp(W x' - |x'|^2/2) / sqrt(m), x' = scale * x, W [m][d] bf16.  A state (S [m][d],
// z [m]) is kept with a log-scale c: the true state is exp(c) * (S, z), so that the stored
// values stay within fp32 range whatever the exponents; c = -inf with S = z = 0 is the empty
// state.  State record of the internal partials: S, z, c, then 3 unused floats.
constexpr int64_t favor_rec(int d, int m) { return (int64_t)m * d + m + 4; }
// (d, m) pairs with kernels: m * d <= 16384, m a multiple of 64
constexpr bool favor_supported(int64_t d, int64_t m) {
  return (d == 64 && (m == 64 || m == 128 || m == 256)) || (d == 128 && (m == 64 || m == 128));
}
constexpr int kFavorTile = 64;        // favor_kv_state: tokens per tile
constexpr int64_t kFavorQueries = 2048;  // favor_out: queries per workgroup

struct FavorStateArgs {
  const void* k;
  const void* v;
  const void* w;
  float* partials;      // [groups][slices][favor_rec]
  int64_t n;            // tokens per head
  int64_t group_len;    // tokens per group (the last group of a head may be shorter)
  int64_t groups_per_head;
  int64_t groups;
  int64_t slices;       // workgroups per group
  int64_t slice_len;    // tokens per workgroup (multiple of kFavorTile)
  float scale;
};

struct FavorReduceArgs {
  const float* partials;  // [groups][slices][favor_rec]
  float* state;           // [groups][favor_rec]
  int64_t groups;
  int64_t slices;
};

struct FavorOutArgs {
  const void* q;
  const void* w;
  void* out;
  const float* state;     // [bh][favor_rec]
  int64_t n;
  int64_t bh;
  float scale;
};

struct FavorDecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* w;
  float* S;               // [bh][m][d]
  float* z;               // [bh][m]
  float* c;               // [bh]
  void* out;
  int64_t bh;
  float scale;
};

struct FavorCausalArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* w;
  void* out;
  const float* seg_state;  // [bh][segs-1][seg_parts][favor_rec]: the leading segments' sums (or null)
  int64_t seg_parts;
  float* sn;               // [bh][m][d], [bh][m], [bh]: the state after token n-1 with its
  float* zn;               //   log-scale (all null: not written)
  float* cn;
  int64_t n;
  int64_t bh;
  int64_t segs;            // segments per head
  int64_t seg_len;         // tokens per segment (multiple of the chunk)
  float scale;
};
// favor_causal chunks: 64 tokens, or 128 where phi(K_c), S^T, one V tile and W fit in LDS
constexpr bool favor_chunk_ok(int64_t d, int64_t m, int64_t chunk) {
  return favor_supported(d, m) && (chunk == 64 || (chunk == 128 && m <= 128));
}

hipError_t launch_favor_kv_state(const FavorStateArgs& a, int d, int m, hipStream_t s);
hipError_t launch_favor_reduce(const FavorReduceArgs& a, int d, int m, hipStream_t s);
hipError_t launch_favor_out(const FavorOutArgs& a, int d, int m, hipStream_t s);
hipError_t launch_favor_decode(const FavorDecodeArgs& a, int d, int m, hipStream_t s);
hipError_t launch_favor_causal(const FavorCausalArgs& a, int d, int m, int chunk, hipStream_t s);
// sn, zn, cn = the empty state (zeros, c = -inf) for every head
hipError_t launch_favor_empty_state(const FavorCausalArgs& a, int d, int m, hipStream_t s);

// Queries per workgroup of the non-causal output kernels.  fp32: 4 waves x 512.  bf16 at
// d = 128: 4 waves x 1024; its workgroups fit only two per compute unit (LDS), so 128 heads x
// 16K queries are one round of workgroups.  bf16 at d = 64: 256.  Its workgroups are then short
// and start in address order, so the rows being written at any moment lie close together, which
// this device's HBM absorbed faster than a thousand long-lived workgroups each writing its own
// 256 KB (128 heads of 16K tokens: 105 -> 93 us).  The fp32 and d = 128 kernels measured no gain
// from smaller tiles.
constexpr int64_t nc_queries(int d, int dtype) { return dtype == 1 ? (d == 128 ? 4096 : 256) : 2048; }

// Tile sizes the host needs for workspace planning.
constexpr int kStateTileBf16 = 64;  // kv_state_bf16: tokens per workgroup tile
constexpr int kStateTileWave = 32;  // kv_state_bf16_waves (D = 64): tokens per wave tile
inline int64_t kv_state_tile(int d, int dtype) {
  return dtype == 1 ? (d == 64 ? 4 * kStateTileWave : kStateTileBf16) : 64;
}

}  // namespace la
