// la_api.hip -- the C ABI declared in include/linattn.h: argument validation, workspace
// planning and kernel dispatch.  Validation happens before any launch; on an error nothing is
// written.  The library allocates nothing and keeps no state between calls.
#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "la_kernels.h"
#include "linattn.h"

// Device memory of la_forward_noncausal_noalloc (see scratch_address below).
static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

namespace {

// Stage-1 workgroups to aim for: the stage-1 kernel's workgroup slots on 256 compute units.  Its
// four-wave workgroups fit two per CU (registers or LDS), four for the fp32 kernel at d = 64
// (90 registers, 40 KB of LDS).
constexpr int64_t state_blocks_target(int d, int dtype) { return (dtype == LA_DTYPE_F32 && d == 64) ? 1024 : 512; }
constexpr int64_t kTargetFavorStateBlocks = 512;  // FAVOR+ stage-1 workgroups to aim for (2 per CU)
constexpr int64_t kTargetCausalBlocks = 256;  // one causal workgroup per compute unit
constexpr int64_t kMaxSegments = 16;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t clamp64(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

int elem_bytes(int dtype) { return dtype == LA_DTYPE_BF16 ? 2 : 4; }

// Checks common to every entry point; fills total bytes of one [B][H][n][d] tensor.
int check_shape(int64_t B, int64_t H, int64_t n, int64_t d, int dtype, int64_t* bh, size_t* bytes) {
  if (dtype != LA_DTYPE_F32 && dtype != LA_DTYPE_BF16) return LA_ERR_DTYPE;
  if (B < 0 || H < 0 || n < 0 || d < 0) return LA_ERR_SHAPE;
  if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
  int64_t t = 0, e = 0;
  if (__builtin_mul_overflow(B, H, &t)) return LA_ERR_SHAPE;
  *bh = t;
  if (__builtin_mul_overflow(t, n, &e) || __builtin_mul_overflow(e, d, &e) ||
      __builtin_mul_overflow(e, (int64_t)elem_bytes(dtype), &e))
    return LA_ERR_SHAPE;
  *bytes = (size_t)e;
  return LA_OK;
}

// Stage-1 plan: `groups` token ranges of `group_len` tokens, each split over `slices`
// workgroups of `slice_len` tokens.  With several slices the kernel writes per-slice partials
// (scratch of groups * slices states) that state_reduce, or the causal kernel, adds up.
struct StatePlan {
  int64_t groups = 0, slices = 0, slice_len = 0;
  size_t scratch_bytes = 0;
};

StatePlan plan_state(int64_t groups, int64_t group_len, int d, int dtype) {
  StatePlan p;
  p.groups = groups;
  const int64_t tile = la::kv_state_tile(d, dtype);
  const int64_t tiles = cdiv(group_len, tile);
  int64_t slices = clamp64(cdiv(state_blocks_target(d, dtype), groups), 1, tiles);
  p.slice_len = cdiv(tiles, slices) * tile;
  p.slices = cdiv(group_len, p.slice_len);
  const size_t E = (size_t)(d * d + d) * sizeof(float);
  p.scratch_bytes = p.slices > 1 ? (size_t)groups * (size_t)p.slices * E : 0;
  return p;
}

size_t state_bytes(int64_t groups, int d) { return (size_t)groups * (size_t)(d * d + d) * sizeof(float); }

// Stage 2 of the non-causal form.  The bf16 output kernel at d = 64 takes 256 queries per
// workgroup (la::nc_queries): adding a head's slice partials in every one of its workgroups would
// re-read them for every 32 KB of queries, so state_reduce adds them once per head, in slice
// order (the same sums, bit for bit), and the output kernel reads one state.  The other output
// kernels take 2048 or 4096 queries and add the partials themselves.
constexpr bool nc_reduce_first(int d, int dtype) { return dtype == LA_DTYPE_BF16 && d == 64; }

// Non-causal workspace: the per-slice partials (and the summed states where they are reduced
// first), or the states themselves when every head has one slice.
size_t nc_ws_bytes(const StatePlan& p, int d, int dtype) {
  if (p.slices == 1) return state_bytes(p.groups, d);
  return p.scratch_bytes + (nc_reduce_first(d, dtype) ? state_bytes(p.groups, d) : 0);
}

// Causal workspace: the leading segments' partials (or their sums when one slice each).
size_t causal_ws_bytes(const StatePlan& p, int d) {
  return p.slices > 1 ? p.scratch_bytes : state_bytes(p.groups, d);
}

// Tokens per segment: enough segments that the (head, segment) workgroups fill every compute
// unit (at most kMaxSegments per head).  Every chunked causal kernel, bf16 or fp32, runs one
// eight-wave workgroup per CU (registers and LDS).
int64_t causal_seg_len(int64_t bh, int64_t n, int64_t chunk) {
  const int64_t nchunks = cdiv(n, chunk);
  int64_t segs = clamp64(cdiv(kTargetCausalBlocks, bh), 1, kMaxSegments);
  segs = clamp64(segs, 1, nchunks);
  return cdiv(nchunks, segs) * chunk;
}

la::KvStateArgs state_args(const StatePlan& p, const void* k, const void* v, float* partials,
                           float* states, int64_t n, int64_t group_len, int64_t groups_per_head) {
  la::KvStateArgs a;
  a.k = k;
  a.v = v;
  a.partials = partials;
  a.state = states;
  a.n = n;
  a.group_len = group_len;
  a.groups_per_head = groups_per_head;
  a.groups = p.groups;
  a.slices = p.slices;
  a.slice_len = p.slice_len;
  return a;
}

bool grid_ok(int64_t blocks) { return blocks > 0 && blocks <= (int64_t)INT_MAX; }

int check_causal(int64_t B, int64_t H, int64_t n, int64_t d, int64_t chunk, int dtype,
                 int64_t* bh, size_t* bytes) {
  int st = check_shape(B, H, n, d, dtype, bh, bytes);
  if (st != LA_OK) return st;
  if (chunk != 64 && chunk != 128) return LA_ERR_UNSUPPORTED;
  if (dtype == LA_DTYPE_F32 && d * chunk > 8192) return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

// A variable-length batch: validates the host offsets and fills the kernels' head table, the
// longest sequence, the head count nseq * H and the bytes of one [sum_s H n_s d] tensor.
struct Varlen {
  la::SeqTable tab;
  int64_t maxn = 0, bh = 0;
  size_t bytes = 0;
};

int make_varlen(const int64_t* cu, int64_t nseq, int64_t H, int64_t d, int dtype, Varlen* v) {
  if (dtype != LA_DTYPE_F32 && dtype != LA_DTYPE_BF16) return LA_ERR_DTYPE;
  if (nseq < 0 || H < 0 || d < 0) return LA_ERR_SHAPE;
  if (d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
  if (nseq > la::kMaxSeqs) return LA_ERR_UNSUPPORTED;
  if (!cu) return LA_ERR_NULL;
  if (cu[0] != 0) return LA_ERR_SHAPE;
  memset(&v->tab, 0, sizeof(v->tab));
  v->tab.heads = H;
  v->tab.cu[0] = 0;
  v->maxn = 0;
  for (int64_t s = 0; s < nseq; ++s) {
    if (cu[s + 1] < cu[s]) return LA_ERR_SHAPE;
    const int64_t ns = cu[s + 1] - cu[s];
    v->maxn = ns > v->maxn ? ns : v->maxn;
    v->tab.cu[s + 1] = cu[s + 1];
  }
  int64_t e = 0;
  if (__builtin_mul_overflow(nseq, H, &v->bh) || __builtin_mul_overflow(H, cu[nseq], &e) ||
      __builtin_mul_overflow(e, d, &e) || __builtin_mul_overflow(e, (int64_t)elem_bytes(dtype), &e))
    return LA_ERR_SHAPE;
  v->bytes = (size_t)e;
  return LA_OK;
}

// ---- FAVOR+ (positive random features)
int check_favor(int64_t B, int64_t H, int64_t n, int64_t d, int64_t m, int dtype, int64_t* bh,
                size_t* bytes) {
  int st = check_shape(B, H, n, d, dtype, bh, bytes);
  if (st != LA_OK) return st;
  if (m < 0) return LA_ERR_SHAPE;
  if (dtype != LA_DTYPE_BF16 || !la::favor_supported(d, m)) return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

bool scale_ok(float scale) { return scale > 0.f && scale <= 3.0e38f; }  // positive and finite

// Stage-1 plan of the FAVOR+ state sums: groups of group_len tokens, each over `slices`
// workgroups (at most 64, the reduction's limit) of a multiple of the tile.
StatePlan plan_favor_state(int64_t groups, int64_t group_len, int d, int m) {
  StatePlan p;
  p.groups = groups;
  const int64_t tiles = cdiv(group_len, la::kFavorTile);
  const int64_t slices = clamp64(cdiv(kTargetFavorStateBlocks, groups), 1, tiles < 64 ? tiles : 64);
  p.slice_len = cdiv(tiles, slices) * la::kFavorTile;
  p.slices = cdiv(group_len, p.slice_len);
  p.scratch_bytes = (size_t)groups * (size_t)p.slices * (size_t)la::favor_rec(d, m) * sizeof(float);
  return p;
}

// Non-causal FAVOR+ workspace: the per-slice partial records, then one record per head.
size_t favor_nc_ws_bytes(const StatePlan& p, int d, int m) {
  return round256(p.scratch_bytes) + (size_t)p.groups * (size_t)la::favor_rec(d, m) * sizeof(float);
}

// Causal FAVOR+ plan: segments per head as for elu + 1 (chunk 64); the leading segments' state
// sums need the workspace.
struct FavorCausalPlan {
  int64_t seg_len = 0, segs = 0;
  StatePlan st;
  size_t ws = 0;
};

FavorCausalPlan plan_favor_causal(int64_t bh, int64_t n, int d, int m, int64_t chunk) {
  FavorCausalPlan p;
  p.seg_len = causal_seg_len(bh, n, chunk);
  p.segs = cdiv(n, p.seg_len);
  if (p.segs > 1) {
    p.st = plan_favor_state(bh * (p.segs - 1), p.seg_len, d, m);
    p.ws = p.st.scratch_bytes;
  }
  return p;
}

// The non-causal call's checks that do not involve the workspace (same order for both entry
// points that take one), its plan and the bytes of one [B][H][n][d] tensor.
struct NcCall {
  int64_t bh = 0;
  size_t bytes = 0;
  StatePlan plan;
  size_t need = 0;
};

int check_noncausal(const void* q, const void* k, const void* v, void* out, int64_t B, int64_t H,
                    int64_t n, int64_t d, int dtype, NcCall* c) {
  int st = check_shape(B, H, n, d, dtype, &c->bh, &c->bytes);
  if (st != LA_OK) return st;
  if (c->bh == 0 || n == 0) return LA_OK;
  if (!q || !k || !v || !out) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return LA_ERR_ALIGN;
  c->plan = plan_state(c->bh, n, (int)d, dtype);
  c->need = nc_ws_bytes(c->plan, (int)d, dtype);
  if (overlaps(out, c->bytes, q, c->bytes) || overlaps(out, c->bytes, k, c->bytes) ||
      overlaps(out, c->bytes, v, c->bytes))
    return LA_ERR_ALIAS;
  if (!grid_ok(c->plan.groups * c->plan.slices) || !grid_ok(c->bh * cdiv(n, la::nc_queries((int)d, dtype))))
    return LA_ERR_SHAPE;
  return LA_OK;
}

// Stage 1, the reduction where it applies, and the output kernel on `s`, with the workspace `ws`
// (nc_ws_bytes(p, d, dtype) bytes, validated by the caller): partials first, then the summed
// states.  n is the (longest) sequence length; tab the variable-length table or null.
int run_nc_stages(const StatePlan& p, const void* q, const void* k, const void* v, void* out, int64_t n,
                  int64_t bh, int d, int dtype, void* ws, hipStream_t s, const la::SeqTable* tab) {
  float* parts = reinterpret_cast<float*>(ws);
  const bool reduce = p.slices > 1 && nc_reduce_first(d, dtype);
  float* states = reduce ? parts + p.scratch_bytes / sizeof(float) : parts;
  la::KvStateArgs ka = state_args(p, k, v, parts, states, n, n, 1);
  if (la::launch_kv_state(ka, d, dtype, s, tab) != hipSuccess) return LA_ERR_HIP;
  if (reduce && la::launch_state_reduce(ka, d, s) != hipSuccess) return LA_ERR_HIP;
  la::NcOutArgs oa;  // otherwise the output kernel adds each head's slices itself
  oa.q = q;
  oa.out = out;
  oa.state = states;
  oa.slices = reduce ? 1 : p.slices;
  oa.n = n;
  oa.bh = bh;
  if (la::launch_nc_out(oa, d, dtype, s, tab) != hipSuccess) return LA_ERR_HIP;
  return LA_OK;
}

// Both stages on `stream` (c.need bytes of workspace, validated by the caller).
int run_noncausal(const NcCall& c, const void* q, const void* k, const void* v, void* out, int64_t n,
                  int d, int dtype, void* ws, void* stream) {
  return run_nc_stages(c.plan, q, k, v, out, n, c.bh, d, dtype, ws, reinterpret_cast<hipStream_t>(stream),
                       nullptr);
}

// ---- scratch of la_forward_noncausal_noalloc
// One array per GPU, reserved when the library's code is loaded on that GPU and held until the
// process ends.  On the host, `scratch` names a stand-in, not device memory: host code takes the
// array's device address from hipGetSymbolAddress, once per device (with that device current),
// and passes only that address on.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not looked up)

int scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return LA_OK;
}

}  // namespace

extern "C" {

int la_abi_version(void) { return LA_ABI_VERSION; }

const char* la_status_string(int status) {
  switch (status) {
    case LA_OK: return "ok";
    case LA_ERR_NULL: return "a required pointer is NULL";
    case LA_ERR_SHAPE: return "invalid (negative or overflowing) shape";
    case LA_ERR_DTYPE: return "unknown element type";
    case LA_ERR_UNSUPPORTED: return "unsupported head dimension, chunk or dtype combination";
    case LA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case LA_ERR_WORKSPACE: return "workspace missing or too small";
    case LA_ERR_ALIAS: return "output overlaps an input, the state or the workspace";
    case LA_ERR_HIP: return "HIP kernel launch failed";
    case LA_ERR_VALUE: return "invalid scalar argument (scale must be positive and finite)";
    default: return "unknown status";
  }
}

size_t la_noncausal_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, la_dtype_t dtype) {
  int64_t bh = 0;
  size_t bytes = 0;
  if (check_shape(B, H, n, d, dtype, &bh, &bytes) != LA_OK) return 0;
  if (bh == 0 || n == 0) return 0;
  return nc_ws_bytes(plan_state(bh, n, (int)d, dtype), (int)d, dtype);
}

int la_forward_noncausal(const void* q, const void* k, const void* v, void* out, int64_t B,
                         int64_t H, int64_t n, int64_t d, la_dtype_t dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
  NcCall c;
  int st = check_noncausal(q, k, v, out, B, H, n, d, dtype, &c);
  if (st != LA_OK || c.bh == 0 || n == 0) return st;
  if (!workspace || workspace_bytes < c.need) return LA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LA_ERR_ALIGN;
  if (overlaps(out, c.bytes, workspace, c.need)) return LA_ERR_ALIAS;
  return run_noncausal(c, q, k, v, out, n, (int)d, dtype, workspace, stream);
}

int la_forward_noncausal_noalloc(const void* q, const void* k, const void* v, void* out, int64_t B,
                                 int64_t H, int64_t n, int64_t d, la_dtype_t dtype, void* stream) {
  NcCall c;
  int st = check_noncausal(q, k, v, out, B, H, n, d, dtype, &c);
  if (st != LA_OK || c.bh == 0 || n == 0) return st;
  if (c.need > LA_NOALLOC_SCRATCH_BYTES) return LA_ERR_WORKSPACE;  // before any HIP call
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != LA_OK) return st;
  if (overlaps(out, c.bytes, ws, c.need)) return LA_ERR_ALIAS;
  return run_noncausal(c, q, k, v, out, n, (int)d, dtype, ws, stream);
}

size_t la_causal_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, int64_t chunk,
                                 la_dtype_t dtype) {
  int64_t bh = 0;
  size_t bytes = 0;
  if (check_causal(B, H, n, d, chunk, dtype, &bh, &bytes) != LA_OK) return 0;
  if (bh == 0 || n == 0) return 0;
  const int64_t seg_len = causal_seg_len(bh, n, chunk);
  const int64_t segs = cdiv(n, seg_len);
  if (segs == 1) return 0;
  return causal_ws_bytes(plan_state(bh * (segs - 1), seg_len, (int)d, dtype), (int)d);
}

int la_causal_plan(int64_t B, int64_t H, int64_t n, int64_t d, int64_t chunk, la_dtype_t dtype,
                   int64_t* seg_len) {
  int64_t bh = 0;
  size_t bytes = 0;
  int st = check_causal(B, H, n, d, chunk, dtype, &bh, &bytes);
  if (st != LA_OK) return st;
  if (!seg_len) return LA_ERR_NULL;
  *seg_len = (bh == 0 || n == 0) ? chunk : causal_seg_len(bh, n, chunk);
  return LA_OK;
}

size_t la_state_sums_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, la_dtype_t dtype,
                                     int64_t seg_len, int64_t nseg) {
  int64_t bh = 0;
  size_t bytes = 0;
  if (check_shape(B, H, n, d, dtype, &bh, &bytes) != LA_OK) return 0;
  if (bh == 0 || n == 0 || seg_len < 1 || nseg < 1) return 0;
  return plan_state(bh * nseg, seg_len, (int)d, dtype).scratch_bytes;
}

int la_state_sums(const void* k, const void* v, float* sums, int64_t B, int64_t H, int64_t n,
                  int64_t d, la_dtype_t dtype, int64_t seg_len, int64_t nseg, void* workspace,
                  size_t workspace_bytes, void* stream) {
  int64_t bh = 0;
  size_t bytes = 0;
  int st = check_shape(B, H, n, d, dtype, &bh, &bytes);
  if (st != LA_OK) return st;
  if (seg_len < 1 || nseg < 1) return LA_ERR_SHAPE;
  if (bh == 0 || n == 0) return LA_OK;
  int64_t last = 0;
  if (__builtin_mul_overflow(nseg - 1, seg_len, &last) || last >= n) return LA_ERR_SHAPE;
  if (!k || !v || !sums) return LA_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(sums)) return LA_ERR_ALIGN;
  const StatePlan p = plan_state(bh * nseg, seg_len, (int)d, dtype);
  if (p.scratch_bytes > 0) {
    if (!workspace || workspace_bytes < p.scratch_bytes) return LA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return LA_ERR_ALIGN;
  }
  const size_t sbytes = state_bytes(p.groups, (int)d);
  if (overlaps(sums, sbytes, k, bytes) || overlaps(sums, sbytes, v, bytes) ||
      overlaps(sums, sbytes, workspace, p.scratch_bytes))
    return LA_ERR_ALIAS;
  if (!grid_ok(p.groups * p.slices)) return LA_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  la::KvStateArgs ka = state_args(p, k, v, reinterpret_cast<float*>(workspace), sums, n, seg_len, nseg);
  if (la::launch_kv_state(ka, (int)d, dtype, s) != hipSuccess) return LA_ERR_HIP;
  if (p.slices > 1 && la::launch_state_reduce(ka, (int)d, s) != hipSuccess) return LA_ERR_HIP;
  return LA_OK;
}

int la_causal_segments(const void* q, const void* k, const void* v, void* out,
                       const float* sums, int64_t B, int64_t H, int64_t n, int64_t d,
                       int64_t chunk, la_dtype_t dtype, int64_t seg_len, void* stream) {
  int64_t bh = 0;
  size_t bytes = 0;
  int st = check_causal(B, H, n, d, chunk, dtype, &bh, &bytes);
  if (st != LA_OK) return st;
  if (seg_len < chunk || seg_len % chunk != 0) return LA_ERR_SHAPE;
  if (bh == 0 || n == 0) return LA_OK;
  const int64_t segs = cdiv(n, seg_len);
  if (!q || !k || !v || !out || (segs > 1 && !sums)) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (sums && !aligned16(sums)))
    return LA_ERR_ALIGN;
  const size_t sbytes = (size_t)bh * (size_t)(segs - 1) * (size_t)(d * d + d) * sizeof(float);
  if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) ||
      overlaps(out, bytes, v, bytes) || overlaps(out, bytes, sums, sbytes))
    return LA_ERR_ALIAS;
  if (!grid_ok(bh * segs)) return LA_ERR_SHAPE;
  la::CausalArgs ca;
  ca.q = q;
  ca.k = k;
  ca.v = v;
  ca.out = out;
  ca.seg_state = segs > 1 ? sums : nullptr;
  ca.seg_parts = 1;
  ca.s0 = ca.z0 = nullptr;
  ca.sn = ca.zn = nullptr;
  ca.n = n;
  ca.bh = bh;
  ca.segs = segs;
  ca.seg_len = seg_len;
  if (la::launch_causal(ca, (int)d, (int)chunk, dtype, reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return LA_ERR_HIP;
  return LA_OK;
}

int la_forward_causal(const void* q, const void* k, const void* v, void* out, int64_t B,
                      int64_t H, int64_t n, int64_t d, int64_t chunk, la_dtype_t dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return la_forward_causal_state(q, k, v, out, nullptr, nullptr, nullptr, nullptr, B, H, n, d,
                                 chunk, dtype, workspace, workspace_bytes, stream);
}

int la_forward_causal_state(const void* q, const void* k, const void* v, void* out,
                            const float* S0, const float* z0, float* Sn, float* zn, int64_t B,
                            int64_t H, int64_t n, int64_t d, int64_t chunk, la_dtype_t dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  int64_t bh = 0;
  size_t bytes = 0;
  int st = check_causal(B, H, n, d, chunk, dtype, &bh, &bytes);
  if (st != LA_OK) return st;
  if (!S0 != !z0 || !Sn != !zn) return LA_ERR_NULL;  // each state is given whole or not at all
  if (bh == 0) return LA_OK;
  const size_t sbytes = (size_t)bh * (size_t)(d * d) * sizeof(float);
  const size_t zbytes = (size_t)bh * (size_t)d * sizeof(float);
  if ((S0 && (!aligned16(S0) || !aligned16(z0))) || (Sn && (!aligned16(Sn) || !aligned16(zn))))
    return LA_ERR_ALIGN;
  if (Sn && (overlaps(Sn, sbytes, zn, zbytes) || overlaps(Sn, sbytes, S0, sbytes) ||
             overlaps(Sn, sbytes, z0, zbytes) || overlaps(zn, zbytes, S0, sbytes) ||
             overlaps(zn, zbytes, z0, zbytes)))
    return LA_ERR_ALIAS;
  la::CausalArgs ca;
  ca.q = q;
  ca.k = k;
  ca.v = v;
  ca.out = out;
  ca.seg_state = nullptr;
  ca.seg_parts = 1;
  ca.s0 = S0;
  ca.z0 = z0;
  ca.sn = Sn;
  ca.zn = zn;
  ca.n = n;
  ca.bh = bh;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (n == 0) {  // no tokens: the final state is the initial one
    if (Sn && la::launch_state_copy(ca, (int)d, s) != hipSuccess) return LA_ERR_HIP;
    return LA_OK;
  }
  if (!q || !k || !v || !out) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return LA_ERR_ALIGN;
  const int64_t seg_len = causal_seg_len(bh, n, chunk);
  const int64_t segs = cdiv(n, seg_len);
  StatePlan p;
  size_t need = 0;
  if (segs > 1) {
    p = plan_state(bh * (segs - 1), seg_len, (int)d, dtype);
    need = causal_ws_bytes(p, (int)d);
    if (!workspace || workspace_bytes < need) return LA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return LA_ERR_ALIGN;
  }
  if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) ||
      overlaps(out, bytes, v, bytes) || overlaps(out, bytes, workspace, need) ||
      overlaps(out, bytes, S0, sbytes) || overlaps(out, bytes, z0, zbytes) ||
      overlaps(out, bytes, Sn, sbytes) || overlaps(out, bytes, zn, zbytes))
    return LA_ERR_ALIAS;
  if (Sn && (overlaps(Sn, sbytes, q, bytes) || overlaps(Sn, sbytes, k, bytes) ||
             overlaps(Sn, sbytes, v, bytes) || overlaps(Sn, sbytes, workspace, need) ||
             overlaps(zn, zbytes, q, bytes) || overlaps(zn, zbytes, k, bytes) ||
             overlaps(zn, zbytes, v, bytes) || overlaps(zn, zbytes, workspace, need)))
    return LA_ERR_ALIAS;
  if (S0 && (overlaps(S0, sbytes, workspace, need) || overlaps(z0, zbytes, workspace, need)))
    return LA_ERR_ALIAS;
  if (!grid_ok(bh * segs) || (segs > 1 && !grid_ok(p.groups * p.slices))) return LA_ERR_SHAPE;
  ca.segs = segs;
  ca.seg_len = seg_len;
  if (segs > 1) {
    // the chunked kernel adds the leading segments' slice partials itself
    float* parts = reinterpret_cast<float*>(workspace);
    la::KvStateArgs ka = state_args(p, k, v, parts, parts, n, seg_len, segs - 1);
    if (la::launch_kv_state(ka, (int)d, dtype, s) != hipSuccess) return LA_ERR_HIP;
    ca.seg_state = parts;
    ca.seg_parts = p.slices;
  }
  if (la::launch_causal(ca, (int)d, (int)chunk, dtype, s) != hipSuccess) return LA_ERR_HIP;
  return LA_OK;
}

static int decode_step(const void* q, const void* k, const void* v, float* S, float* z, void* out,
                       const uint8_t* active, int64_t B, int64_t H, int64_t d, la_dtype_t dtype, void* stream) {
  int64_t bh = 0;
  size_t bytes = 0;
  int st = check_shape(B, H, 1, d, dtype, &bh, &bytes);
  if (st != LA_OK) return st;
  if (bh == 0) return LA_OK;
  if (!q || !k || !v || !S || !z || !out) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(S) || !aligned16(z) ||
      !aligned16(out))
    return LA_ERR_ALIGN;
  const size_t sbytes = (size_t)bh * (size_t)(d * d) * sizeof(float);
  const size_t zbytes = (size_t)bh * (size_t)d * sizeof(float);
  // S and z are written in place while other workgroups still read q, k and v
  const void* ins[3] = {q, k, v};
  for (int i = 0; i < 3; ++i)
    if (overlaps(out, bytes, ins[i], bytes) || overlaps(S, sbytes, ins[i], bytes) ||
        overlaps(z, zbytes, ins[i], bytes))
      return LA_ERR_ALIAS;
  if (overlaps(out, bytes, S, sbytes) || overlaps(out, bytes, z, zbytes) || overlaps(S, sbytes, z, zbytes))
    return LA_ERR_ALIAS;
  if (active && (overlaps(active, (size_t)B, out, bytes) || overlaps(active, (size_t)B, S, sbytes) ||
                 overlaps(active, (size_t)B, z, zbytes)))
    return LA_ERR_ALIAS;
  if (!grid_ok(bh)) return LA_ERR_SHAPE;
  la::DecodeArgs da;
  da.q = q;
  da.k = k;
  da.v = v;
  da.S = S;
  da.z = z;
  da.out = out;
  da.active = active;
  da.heads = H;
  da.bh = bh;
  if (la::launch_decode(da, (int)d, dtype, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return LA_ERR_HIP;
  return LA_OK;
}

int la_decode_step(const void* q, const void* k, const void* v, float* S, float* z, void* out,
                   int64_t B, int64_t H, int64_t d, la_dtype_t dtype, void* stream) {
  return decode_step(q, k, v, S, z, out, nullptr, B, H, d, dtype, stream);
}

int la_decode_step_masked(const void* q, const void* k, const void* v, float* S, float* z,
                          void* out, const uint8_t* active, int64_t B, int64_t H, int64_t d,
                          la_dtype_t dtype, void* stream) {
  int64_t bh = 0;
  size_t bytes = 0;
  const int st = check_shape(B, H, 1, d, dtype, &bh, &bytes);  // B * H is known not to overflow
  if (st != LA_OK) return st;
  if (!active && bh > 0) return LA_ERR_NULL;
  return decode_step(q, k, v, S, z, out, active, B, H, d, dtype, stream);
}

size_t la_noncausal_varlen_workspace_bytes(const int64_t* cu_seqlens, int64_t nseq, int64_t H,
                                           int64_t d, la_dtype_t dtype) {
  Varlen vl;
  if (make_varlen(cu_seqlens, nseq, H, d, dtype, &vl) != LA_OK || vl.bh == 0 || vl.maxn == 0) return 0;
  return nc_ws_bytes(plan_state(vl.bh, vl.maxn, (int)d, dtype), (int)d, dtype);
}

int la_forward_noncausal_varlen(const void* q, const void* k, const void* v, void* out,
                                const int64_t* cu_seqlens, int64_t nseq, int64_t H, int64_t d,
                                la_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  Varlen vl;
  int st = make_varlen(cu_seqlens, nseq, H, d, dtype, &vl);
  if (st != LA_OK) return st;
  if (vl.bh == 0 || vl.maxn == 0) return LA_OK;
  if (!q || !k || !v || !out) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return LA_ERR_ALIGN;
  const StatePlan p = plan_state(vl.bh, vl.maxn, (int)d, dtype);
  const size_t need = nc_ws_bytes(p, (int)d, dtype);
  if (!workspace || workspace_bytes < need) return LA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LA_ERR_ALIGN;
  const size_t bytes = vl.bytes;
  if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) ||
      overlaps(out, bytes, v, bytes) || overlaps(out, bytes, workspace, need))
    return LA_ERR_ALIAS;
  if (!grid_ok(p.groups * p.slices) || !grid_ok(vl.bh * cdiv(vl.maxn, la::nc_queries((int)d, dtype))))
    return LA_ERR_SHAPE;
  return run_nc_stages(p, q, k, v, out, vl.maxn, vl.bh, (int)d, dtype, workspace,
                       reinterpret_cast<hipStream_t>(stream), &vl.tab);
}

size_t la_causal_varlen_workspace_bytes(const int64_t* cu_seqlens, int64_t nseq, int64_t H,
                                        int64_t d, int64_t chunk, la_dtype_t dtype) {
  Varlen vl;
  if (make_varlen(cu_seqlens, nseq, H, d, dtype, &vl) != LA_OK || vl.bh == 0 || vl.maxn == 0) return 0;
  if (chunk != 64 && chunk != 128) return 0;
  const int64_t seg_len = causal_seg_len(vl.bh, vl.maxn, chunk);
  const int64_t segs = cdiv(vl.maxn, seg_len);
  if (segs == 1) return 0;
  return causal_ws_bytes(plan_state(vl.bh * (segs - 1), seg_len, (int)d, dtype), (int)d);
}

int la_forward_causal_varlen(const void* q, const void* k, const void* v, void* out,
                             const int64_t* cu_seqlens, int64_t nseq, int64_t H, int64_t d,
                             int64_t chunk, la_dtype_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  Varlen vl;
  int st = make_varlen(cu_seqlens, nseq, H, d, dtype, &vl);
  if (st != LA_OK) return st;
  if (chunk != 64 && chunk != 128) return LA_ERR_UNSUPPORTED;
  if (dtype == LA_DTYPE_F32 && d * chunk > 8192) return LA_ERR_UNSUPPORTED;
  if (vl.bh == 0 || vl.maxn == 0) return LA_OK;
  if (!q || !k || !v || !out) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return LA_ERR_ALIGN;
  const int64_t seg_len = causal_seg_len(vl.bh, vl.maxn, chunk);
  const int64_t segs = cdiv(vl.maxn, seg_len);
  StatePlan p;
  size_t need = 0;
  if (segs > 1) {
    p = plan_state(vl.bh * (segs - 1), seg_len, (int)d, dtype);
    need = causal_ws_bytes(p, (int)d);
    if (!workspace || workspace_bytes < need) return LA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return LA_ERR_ALIGN;
  }
  const size_t bytes = vl.bytes;
  if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) ||
      overlaps(out, bytes, v, bytes) || overlaps(out, bytes, workspace, need))
    return LA_ERR_ALIAS;
  if (!grid_ok(vl.bh * segs) || (segs > 1 && !grid_ok(p.groups * p.slices))) return LA_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  la::CausalArgs ca;
  ca.q = q;
  ca.k = k;
  ca.v = v;
  ca.out = out;
  ca.seg_state = nullptr;
  ca.seg_parts = 1;
  ca.s0 = ca.z0 = nullptr;
  ca.sn = ca.zn = nullptr;
  ca.n = vl.maxn;
  ca.bh = vl.bh;
  ca.segs = segs;
  ca.seg_len = seg_len;
  if (segs > 1) {
    float* parts = reinterpret_cast<float*>(workspace);
    la::KvStateArgs ka = state_args(p, k, v, parts, parts, vl.maxn, seg_len, segs - 1);
    if (la::launch_kv_state(ka, (int)d, dtype, s, &vl.tab) != hipSuccess) return LA_ERR_HIP;
    ca.seg_state = parts;
    ca.seg_parts = p.slices;
  }
  if (la::launch_causal(ca, (int)d, (int)chunk, dtype, s, &vl.tab) != hipSuccess) return LA_ERR_HIP;
  return LA_OK;
}

// ---------------------------------------------------------------- FAVOR+
size_t la_favor_noncausal_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, int64_t m,
                                          la_dtype_t dtype) {
  int64_t bh = 0;
  size_t bytes = 0;
  if (check_favor(B, H, n, d, m, dtype, &bh, &bytes) != LA_OK || bh == 0 || n == 0) return 0;
  return favor_nc_ws_bytes(plan_favor_state(bh, n, (int)d, (int)m), (int)d, (int)m);
}

int la_favor_forward_noncausal(const void* q, const void* k, const void* v, const void* w,
                               void* out, int64_t B, int64_t H, int64_t n, int64_t d, int64_t m,
                               float scale, la_dtype_t dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  int64_t bh = 0;
  size_t bytes = 0;
  int st = check_favor(B, H, n, d, m, dtype, &bh, &bytes);
  if (st != LA_OK) return st;
  if (!scale_ok(scale)) return LA_ERR_VALUE;
  if (bh == 0 || n == 0) return LA_OK;
  if (!q || !k || !v || !w || !out) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(w) || !aligned16(out))
    return LA_ERR_ALIGN;
  const StatePlan p = plan_favor_state(bh, n, (int)d, (int)m);
  const size_t need = favor_nc_ws_bytes(p, (int)d, (int)m);
  if (!workspace || workspace_bytes < need) return LA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LA_ERR_ALIGN;
  const size_t wbytes = (size_t)(m * d) * 2;
  if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) ||
      overlaps(out, bytes, v, bytes) || overlaps(out, bytes, w, wbytes) ||
      overlaps(out, bytes, workspace, need))
    return LA_ERR_ALIAS;
  if (!grid_ok(p.groups * p.slices) || !grid_ok(bh * cdiv(n, la::kFavorQueries))) return LA_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  float* parts = reinterpret_cast<float*>(ws);
  float* states = reinterpret_cast<float*>(ws + round256(p.scratch_bytes));
  la::FavorStateArgs ka;
  ka.k = k;
  ka.v = v;
  ka.w = w;
  ka.partials = parts;
  ka.n = n;
  ka.group_len = n;
  ka.groups_per_head = 1;
  ka.groups = bh;
  ka.slices = p.slices;
  ka.slice_len = p.slice_len;
  ka.scale = scale;
  if (la::launch_favor_kv_state(ka, (int)d, (int)m, s) != hipSuccess) return LA_ERR_HIP;
  la::FavorReduceArgs ra;
  ra.partials = parts;
  ra.state = states;
  ra.groups = bh;
  ra.slices = p.slices;
  if (la::launch_favor_reduce(ra, (int)d, (int)m, s) != hipSuccess) return LA_ERR_HIP;
  la::FavorOutArgs oa;
  oa.q = q;
  oa.w = w;
  oa.out = out;
  oa.state = states;
  oa.n = n;
  oa.bh = bh;
  oa.scale = scale;
  if (la::launch_favor_out(oa, (int)d, (int)m, s) != hipSuccess) return LA_ERR_HIP;
  return LA_OK;
}

int la_favor_decode_step(const void* q, const void* k, const void* v, const void* w, float* S,
                         float* z, float* c, void* out, int64_t B, int64_t H, int64_t d, int64_t m,
                         float scale, la_dtype_t dtype, void* stream) {
  int64_t bh = 0;
  size_t bytes = 0;
  int st = check_favor(B, H, 1, d, m, dtype, &bh, &bytes);
  if (st != LA_OK) return st;
  if (!scale_ok(scale)) return LA_ERR_VALUE;
  if (bh == 0) return LA_OK;
  if (!q || !k || !v || !w || !S || !z || !c || !out) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(w) || !aligned16(S) ||
      !aligned16(out) || ((uintptr_t)z & 3u) || ((uintptr_t)c & 3u))
    return LA_ERR_ALIGN;
  if (!grid_ok(bh)) return LA_ERR_SHAPE;
  const size_t sb = (size_t)bh * (size_t)(m * d) * sizeof(float);
  const size_t zb = (size_t)bh * (size_t)m * sizeof(float), cb = (size_t)bh * sizeof(float);
  const size_t wbytes = (size_t)(m * d) * 2;
  const void* ins[4] = {q, k, v, w};
  const size_t inb[4] = {bytes, bytes, bytes, wbytes};
  for (int i = 0; i < 4; ++i)
    if (overlaps(out, bytes, ins[i], inb[i]) || overlaps(S, sb, ins[i], inb[i]) ||
        overlaps(z, zb, ins[i], inb[i]) || overlaps(c, cb, ins[i], inb[i]))
      return LA_ERR_ALIAS;
  if (overlaps(out, bytes, S, sb) || overlaps(out, bytes, z, zb) || overlaps(out, bytes, c, cb) ||
      overlaps(S, sb, z, zb) || overlaps(S, sb, c, cb) || overlaps(z, zb, c, cb))
    return LA_ERR_ALIAS;
  la::FavorDecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.w = w;
  a.S = S;
  a.z = z;
  a.c = c;
  a.out = out;
  a.bh = bh;
  a.scale = scale;
  if (la::launch_favor_decode(a, (int)d, (int)m, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return LA_ERR_HIP;
  return LA_OK;
}

size_t la_favor_causal_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, int64_t m,
                                       int64_t chunk, la_dtype_t dtype) {
  int64_t bh = 0;
  size_t bytes = 0;
  if (check_favor(B, H, n, d, m, dtype, &bh, &bytes) != LA_OK || bh == 0 || n == 0) return 0;
  if (!la::favor_chunk_ok(d, m, chunk)) return 0;
  return plan_favor_causal(bh, n, (int)d, (int)m, chunk).ws;
}

int la_favor_forward_causal(const void* q, const void* k, const void* v, const void* w, void* out,
                            float* Sn, float* zn, float* cn, int64_t B, int64_t H, int64_t n,
                            int64_t d, int64_t m, int64_t chunk, float scale, la_dtype_t dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  int64_t bh = 0;
  size_t bytes = 0;
  int st = check_favor(B, H, n, d, m, dtype, &bh, &bytes);
  if (st != LA_OK) return st;
  if (!la::favor_chunk_ok(d, m, chunk)) return LA_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return LA_ERR_VALUE;
  const bool fin = Sn || zn || cn;
  if (fin && !(Sn && zn && cn)) return LA_ERR_NULL;
  if (bh == 0) return LA_OK;
  const size_t sb = (size_t)bh * (size_t)(m * d) * sizeof(float);
  const size_t zb = (size_t)bh * (size_t)m * sizeof(float), cb = (size_t)bh * sizeof(float);
  if (fin) {
    if (!aligned16(Sn) || ((uintptr_t)zn & 3u) || ((uintptr_t)cn & 3u)) return LA_ERR_ALIGN;
    if (overlaps(Sn, sb, zn, zb) || overlaps(Sn, sb, cn, cb) || overlaps(zn, zb, cn, cb)) return LA_ERR_ALIAS;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  la::FavorCausalArgs ca;
  ca.q = q;
  ca.k = k;
  ca.v = v;
  ca.w = w;
  ca.out = out;
  ca.seg_state = nullptr;
  ca.seg_parts = 1;
  ca.sn = Sn;
  ca.zn = zn;
  ca.cn = cn;
  ca.n = n;
  ca.bh = bh;
  ca.segs = 1;
  ca.seg_len = 0;
  ca.scale = scale;
  if (n == 0) {  // no tokens: the final state is the empty state
    if (!fin) return LA_OK;
    if (!grid_ok(bh)) return LA_ERR_SHAPE;
    if (la::launch_favor_empty_state(ca, (int)d, (int)m, s) != hipSuccess) return LA_ERR_HIP;
    return LA_OK;
  }
  if (!q || !k || !v || !w || !out) return LA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(w) || !aligned16(out))
    return LA_ERR_ALIGN;
  const FavorCausalPlan p = plan_favor_causal(bh, n, (int)d, (int)m, chunk);
  if (p.ws > 0) {
    if (!workspace || workspace_bytes < p.ws) return LA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return LA_ERR_ALIGN;
  }
  const size_t wbytes = (size_t)(m * d) * 2;
  const void* ins[4] = {q, k, v, w};
  const size_t inb[4] = {bytes, bytes, bytes, wbytes};
  for (int i = 0; i < 4; ++i) {
    if (overlaps(out, bytes, ins[i], inb[i])) return LA_ERR_ALIAS;
    if (fin && (overlaps(Sn, sb, ins[i], inb[i]) || overlaps(zn, zb, ins[i], inb[i]) ||
                overlaps(cn, cb, ins[i], inb[i])))
      return LA_ERR_ALIAS;
  }
  if (overlaps(out, bytes, workspace, p.ws)) return LA_ERR_ALIAS;
  if (fin && (overlaps(out, bytes, Sn, sb) || overlaps(out, bytes, zn, zb) || overlaps(out, bytes, cn, cb) ||
              overlaps(Sn, sb, workspace, p.ws) || overlaps(zn, zb, workspace, p.ws) ||
              overlaps(cn, cb, workspace, p.ws)))
    return LA_ERR_ALIAS;
  if (!grid_ok(bh * p.segs) || (p.segs > 1 && !grid_ok(p.st.groups * p.st.slices))) return LA_ERR_SHAPE;
  ca.segs = p.segs;
  ca.seg_len = p.seg_len;
  if (p.segs > 1) {
    float* parts = reinterpret_cast<float*>(workspace);
    la::FavorStateArgs ka;
    ka.k = k;
    ka.v = v;
    ka.w = w;
    ka.partials = parts;
    ka.n = n;
    ka.group_len = p.seg_len;
    ka.groups_per_head = p.segs - 1;
    ka.groups = p.st.groups;
    ka.slices = p.st.slices;
    ka.slice_len = p.st.slice_len;
    ka.scale = scale;
    if (la::launch_favor_kv_state(ka, (int)d, (int)m, s) != hipSuccess) return LA_ERR_HIP;
    ca.seg_state = parts;
    ca.seg_parts = p.st.slices;
  }
  if (la::launch_favor_causal(ca, (int)d, (int)m, (int)chunk, s) != hipSuccess) return LA_ERR_HIP;
  return LA_OK;
}

}  // extern "C"
