// abi_host.cpp -- the C ABI's host side (argument validation and planning in la_api.hip) under
// AddressSanitizer and UndefinedBehaviorSanitizer, with no GPU (tests/test_sanitizers.py).
//
// la_api.hip is compiled for the host only; this file supplies what the rest of the library and
// the HIP runtime would: kernel launchers that check the plan they are handed (grids, tiles,
// slices and segments covering every token) and record the call, and the few runtime entry
// points the host code uses.  Device pointers are fake addresses that nothing dereferences.
// main() drives every entry point through its error paths and through valid calls on the
// workloads' shapes, and checks the returned codes and which launchers ran.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "la_kernels.h"
#include "linattn.h"

static int g_fail = 0;
static int g_launches = 0;

#define CHECK(cond, ...)                                        \
  do {                                                          \
    if (!(cond)) {                                              \
      printf("FAIL line %d: ", __LINE__);                       \
      printf(__VA_ARGS__);                                      \
      printf("\n");                                             \
      ++g_fail;                                                 \
    }                                                           \
  } while (0)

// ---------------------------------------------------------------- HIP runtime used by the host code
static unsigned char g_scratch_stand_in[256] __attribute__((aligned(256)));
extern "C" {
void** __hipRegisterFatBinary(const void*) {
  static void* handle = nullptr;
  return &handle;
}
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}
}
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** p, const void*) {
  *p = g_scratch_stand_in;
  return hipSuccess;
}

// ---------------------------------------------------------------- launchers: check the plan
namespace la {
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

hipError_t launch_kv_state(const KvStateArgs& a, int d, int dtype, hipStream_t, const SeqTable*) {
  ++g_launches;
  CHECK(d == 64 || d == 128, "kv_state d %d", d);
  CHECK(a.groups > 0 && a.slices > 0 && a.groups * a.slices <= INT32_MAX, "kv_state grid");
  CHECK(a.slice_len > 0 && a.slice_len % kv_state_tile(d, dtype) == 0, "kv_state slice_len %lld",
        (long long)a.slice_len);
  CHECK(a.slices * a.slice_len >= a.group_len, "kv_state slices do not cover the group");
  CHECK(a.groups % a.groups_per_head == 0, "kv_state groups per head");
  CHECK(a.slices == 1 || a.partials != nullptr, "kv_state partials missing");
  return hipSuccess;
}
hipError_t launch_state_reduce(const KvStateArgs& a, int, hipStream_t) {
  ++g_launches;
  CHECK(a.slices > 1 && a.state != nullptr, "state_reduce");
  return hipSuccess;
}
hipError_t launch_nc_out(const NcOutArgs& a, int d, int dtype, hipStream_t, const SeqTable*) {
  ++g_launches;
  CHECK(a.bh > 0 && a.n > 0 && a.slices > 0 && a.state != nullptr, "nc_out args");
  CHECK(a.bh * cdiv(a.n, nc_queries(d, dtype)) <= INT32_MAX, "nc_out grid");
  return hipSuccess;
}
hipError_t launch_causal(const CausalArgs& a, int d, int chunk, int dtype, hipStream_t, const SeqTable*) {
  ++g_launches;
  CHECK(chunk == 64 || chunk == 128, "causal chunk");
  CHECK(dtype == 1 || d * chunk <= 8192, "fp32 causal tile");
  CHECK(a.segs >= 1 && a.seg_len % chunk == 0 && a.seg_len > 0, "causal segments");
  CHECK(a.segs * a.seg_len >= a.n && (a.segs - 1) * a.seg_len < a.n, "segments cover n");
  CHECK(a.segs == 1 || (a.seg_state != nullptr && a.seg_parts >= 1), "segment sums missing");
  CHECK(!a.s0 == !a.z0 && !a.sn == !a.zn, "state pairs");
  return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs& a, int d, int, hipStream_t) {
  ++g_launches;
  CHECK(a.bh > 0 && (d == 64 || d == 128) && a.heads > 0, "decode args");
  return hipSuccess;
}
hipError_t launch_state_copy(const CausalArgs& a, int, hipStream_t) {
  ++g_launches;
  CHECK(a.sn && a.zn && a.bh > 0, "state copy");
  return hipSuccess;
}
hipError_t launch_favor_kv_state(const FavorStateArgs& a, int d, int m, hipStream_t) {
  ++g_launches;
  CHECK(favor_supported(d, m) && a.slices >= 1 && a.slices <= 64, "favor kv_state");
  CHECK(a.slice_len % kFavorTile == 0 && a.slices * a.slice_len >= a.group_len, "favor slices");
  return hipSuccess;
}
hipError_t launch_favor_reduce(const FavorReduceArgs& a, int, int, hipStream_t) {
  ++g_launches;
  CHECK(a.groups > 0 && a.slices > 0, "favor reduce");
  return hipSuccess;
}
hipError_t launch_favor_out(const FavorOutArgs& a, int, int, hipStream_t) {
  ++g_launches;
  CHECK(a.bh > 0 && a.n > 0, "favor out");
  return hipSuccess;
}
hipError_t launch_favor_decode(const FavorDecodeArgs& a, int, int, hipStream_t) {
  ++g_launches;
  CHECK(a.bh > 0, "favor decode");
  return hipSuccess;
}
hipError_t launch_favor_causal(const FavorCausalArgs& a, int d, int m, int chunk, hipStream_t) {
  ++g_launches;
  CHECK(favor_chunk_ok(d, m, chunk) && a.seg_len % chunk == 0, "favor causal");
  CHECK(a.segs * a.seg_len >= a.n && (a.segs - 1) * a.seg_len < a.n, "favor segments cover n");
  return hipSuccess;
}
hipError_t launch_favor_empty_state(const FavorCausalArgs& a, int, int, hipStream_t) {
  ++g_launches;
  CHECK(a.sn && a.zn && a.cn, "favor empty state");
  return hipSuccess;
}
}  // namespace la

// ---------------------------------------------------------------- the calls
// Fake device buffers: 1 TiB apart and 256-byte aligned, so no two overlap at any shape here.
static void* buf(int i) { return reinterpret_cast<void*>((uintptr_t)(i + 1) << 40); }
static float* fbuf(int i) { return reinterpret_cast<float*>(buf(i)); }
static void* off(void* p, size_t bytes) { return reinterpret_cast<char*>(p) + bytes; }
static const size_t kWs = (size_t)1 << 38;

// expect: status code, and whether a launcher must (true) or must not (false) have run
#define EXPECT(call, code, launched)                                                            \
  do {                                                                                          \
    const int before_ = g_launches;                                                             \
    const int st_ = (call);                                                                     \
    CHECK(st_ == (code), "%s returned %d, expected %d", #call, st_, (code));                    \
    CHECK((g_launches > before_) == (launched), "%s: launchers %s", #call,                      \
          (launched) ? "did not run" : "ran on an error path");                                 \
  } while (0)

static const la_dtype_t BF = LA_DTYPE_BF16, F32 = LA_DTYPE_F32;

static void noncausal() {
  auto nc = [](int64_t B, int64_t H, int64_t n, int64_t d, la_dtype_t dt, void* ws = buf(8), size_t wsb = kWs,
               void* out = buf(3)) {
    return la_forward_noncausal(buf(0), buf(1), buf(2), out, B, H, n, d, dt, ws, wsb, nullptr);
  };
  EXPECT(nc(8, 16, 16384, 64, BF), LA_OK, true);
  EXPECT(nc(4, 32, 65536, 128, F32), LA_OK, true);
  EXPECT(nc(1, 1, 1, 64, BF), LA_OK, true);
  EXPECT(nc(1, 1, 0, 64, BF), LA_OK, false);
  EXPECT(nc(1, 1, 8, 64, (la_dtype_t)7), LA_ERR_DTYPE, false);
  EXPECT(nc(1 << 30, 1 << 30, 1 << 30, 128, BF), LA_ERR_SHAPE, false);
  EXPECT(nc(INT64_MAX, 2, 1, 64, BF), LA_ERR_SHAPE, false);
  EXPECT(nc(1, 1, 8, 96, BF), LA_ERR_UNSUPPORTED, false);
  EXPECT(nc(1, 1, 8, 64, BF, nullptr), LA_ERR_WORKSPACE, false);
  EXPECT(nc(1, 1, 8, 64, BF, buf(8), 16), LA_ERR_WORKSPACE, false);
  EXPECT(nc(1, 1, 8, 64, BF, buf(8), kWs, buf(0)), LA_ERR_ALIAS, false);
  EXPECT(nc(1, 1, 8, 64, BF, buf(8), kWs, off(buf(3), 8)), LA_ERR_ALIGN, false);
  EXPECT(la_forward_noncausal_noalloc(buf(0), buf(1), buf(2), buf(3), 8, 16, 16384, 64, BF, nullptr), LA_OK, true);
  EXPECT(la_forward_noncausal_noalloc(buf(0), buf(1), buf(2), buf(3), 4096, 2, 64, 128, BF, nullptr),
         LA_ERR_WORKSPACE, false);
  CHECK(la_noncausal_workspace_bytes(8, 16, 16384, 64, BF) > 0, "workspace size");
  CHECK(la_noncausal_workspace_bytes(-1, 16, 16384, 64, BF) == 0, "workspace size of a bad shape");
}

static void causal() {
  auto ca = [](int64_t B, int64_t H, int64_t n, int64_t d, int64_t chunk, la_dtype_t dt, void* ws = buf(8)) {
    return la_forward_causal(buf(0), buf(1), buf(2), buf(3), B, H, n, d, chunk, dt, ws, kWs, nullptr);
  };
  EXPECT(ca(4, 32, 65536, 128, 128, BF), LA_OK, true);
  EXPECT(ca(1, 1, 4096, 64, 64, F32), LA_OK, true);
  EXPECT(ca(1, 1, 16 * 128 + 37, 128, 128, BF), LA_OK, true);
  EXPECT(ca(1, 1, 100, 128, 128, F32), LA_ERR_UNSUPPORTED, false);
  EXPECT(ca(1, 1, 100, 64, 96, BF), LA_ERR_UNSUPPORTED, false);
  EXPECT(ca(1, 1, 4096, 64, 64, BF, nullptr), LA_ERR_WORKSPACE, false);
  EXPECT(la_forward_causal_state(buf(0), buf(1), buf(2), buf(3), fbuf(4), fbuf(5), fbuf(6), fbuf(7), 2, 3, 700,
                                 128, 128, BF, buf(8), kWs, nullptr),
         LA_OK, true);
  EXPECT(la_forward_causal_state(nullptr, nullptr, nullptr, nullptr, fbuf(4), fbuf(5), fbuf(6), fbuf(7), 2, 3, 0,
                                 128, 128, BF, nullptr, 0, nullptr),
         LA_OK, true);  // n = 0 hands the state on
  EXPECT(la_forward_causal_state(buf(0), buf(1), buf(2), buf(3), fbuf(4), nullptr, nullptr, nullptr, 1, 1, 8, 64,
                                 64, BF, buf(8), kWs, nullptr),
         LA_ERR_NULL, false);
  EXPECT(la_forward_causal_state(buf(0), buf(1), buf(2), buf(3), fbuf(4), fbuf(5), fbuf(4), fbuf(7), 1, 1, 8, 64,
                                 64, BF, buf(8), kWs, nullptr),
         LA_ERR_ALIAS, false);
  int64_t seg = 0;
  EXPECT(la_causal_plan(4, 32, 65536, 128, 128, BF, &seg), LA_OK, false);
  CHECK(seg == 32768, "C4 plan: seg_len %lld", (long long)seg);
  EXPECT(la_state_sums(buf(1), buf(2), fbuf(4), 4, 32, 65536, 128, BF, seg, 1, buf(8), kWs, nullptr), LA_OK, true);
  EXPECT(la_state_sums(buf(1), buf(2), fbuf(4), 1, 1, 1000, 64, BF, 100, 11, buf(8), kWs, nullptr), LA_ERR_SHAPE,
         false);
  EXPECT(la_causal_segments(buf(0), buf(1), buf(2), buf(3), fbuf(4), 4, 32, 65536, 128, 128, BF, seg, nullptr),
         LA_OK, true);
  EXPECT(la_causal_segments(buf(0), buf(1), buf(2), buf(3), nullptr, 1, 1, 1000, 64, 64, BF, 128, nullptr),
         LA_ERR_NULL, false);
  EXPECT(la_causal_segments(buf(0), buf(1), buf(2), buf(3), fbuf(4), 1, 1, 1000, 64, 64, BF, 100, nullptr),
         LA_ERR_SHAPE, false);
}

static void decode() {
  EXPECT(la_decode_step(buf(0), buf(1), buf(2), fbuf(4), fbuf(5), buf(3), 256, 32, 128, BF, nullptr), LA_OK, true);
  EXPECT(la_decode_step(buf(0), buf(1), buf(2), fbuf(0), fbuf(5), buf(3), 1, 1, 64, BF, nullptr), LA_ERR_ALIAS,
         false);
  const uint8_t* act = reinterpret_cast<const uint8_t*>(buf(9));
  EXPECT(la_decode_step_masked(buf(0), buf(1), buf(2), fbuf(4), fbuf(5), buf(3), act, 256, 32, 128, BF, nullptr),
         LA_OK, true);
  EXPECT(la_decode_step_masked(buf(0), buf(1), buf(2), fbuf(4), fbuf(5), buf(3), nullptr, INT64_MAX, 4, 128, BF,
                               nullptr),
         LA_ERR_SHAPE, false);
  EXPECT(la_decode_step_masked(buf(0), buf(1), buf(2), fbuf(4), fbuf(5), buf(3), nullptr, 2, 4, 128, BF, nullptr),
         LA_ERR_NULL, false);
}

static void varlen() {
  int64_t cu[257];
  cu[0] = 0;
  for (int s = 0; s < 256; ++s) cu[s + 1] = cu[s] + (s * 7919) % 3001;  // 256 sequences, some empty
  size_t ws = la_noncausal_varlen_workspace_bytes(cu, 256, 4, 64, BF);
  CHECK(ws > 0, "varlen workspace");
  EXPECT(la_forward_noncausal_varlen(buf(0), buf(1), buf(2), buf(3), cu, 256, 4, 64, BF, buf(8), kWs, nullptr),
         LA_OK, true);
  EXPECT(la_forward_causal_varlen(buf(0), buf(1), buf(2), buf(3), cu, 256, 4, 128, 128, BF, buf(8), kWs, nullptr),
         LA_OK, true);
  int64_t bad[3] = {0, 5, 3};
  EXPECT(la_forward_noncausal_varlen(buf(0), buf(1), buf(2), buf(3), bad, 2, 4, 64, BF, buf(8), kWs, nullptr),
         LA_ERR_SHAPE, false);
  int64_t many[258];
  for (int s = 0; s < 258; ++s) many[s] = s;
  EXPECT(la_forward_noncausal_varlen(buf(0), buf(1), buf(2), buf(3), many, 257, 4, 64, BF, buf(8), kWs, nullptr),
         LA_ERR_UNSUPPORTED, false);
  EXPECT(la_forward_causal_varlen(buf(0), buf(1), buf(2), buf(3), nullptr, 2, 4, 64, 64, BF, buf(8), kWs, nullptr),
         LA_ERR_NULL, false);
}

static void favor() {
  EXPECT(la_favor_forward_noncausal(buf(0), buf(1), buf(2), buf(10), buf(3), 8, 16, 16384, 64, 256, 0.35f, BF,
                                    buf(8), kWs, nullptr),
         LA_OK, true);
  EXPECT(la_favor_forward_causal(buf(0), buf(1), buf(2), buf(10), buf(3), fbuf(4), fbuf(5), fbuf(6), 4, 32, 65536,
                                 128, 128, 64, 0.3f, BF, buf(8), kWs, nullptr),
         LA_OK, true);
  EXPECT(la_favor_forward_causal(nullptr, nullptr, nullptr, nullptr, nullptr, fbuf(4), fbuf(5), fbuf(6), 2, 2, 0,
                                 64, 128, 64, 0.3f, BF, nullptr, 0, nullptr),
         LA_OK, true);
  EXPECT(la_favor_decode_step(buf(0), buf(1), buf(2), buf(10), fbuf(4), fbuf(5), fbuf(6), buf(3), 256, 32, 128, 128,
                              0.3f, BF, nullptr),
         LA_OK, true);
  EXPECT(la_favor_forward_noncausal(buf(0), buf(1), buf(2), buf(10), buf(3), 1, 1, 8, 64, 256, 0.0f, BF, buf(8),
                                    kWs, nullptr),
         LA_ERR_VALUE, false);
  EXPECT(la_favor_forward_noncausal(buf(0), buf(1), buf(2), buf(10), buf(3), 1, 1, 8, 128, 256, 0.3f, BF, buf(8),
                                    kWs, nullptr),
         LA_ERR_UNSUPPORTED, false);
}

int main() {
  CHECK(la_abi_version() == LA_ABI_VERSION, "abi version");
  for (int st = -10; st <= 0; ++st) CHECK(la_status_string(st) != nullptr, "status string");
  noncausal();
  causal();
  decode();
  varlen();
  favor();
  if (g_fail) {
    printf("%d check(s) failed\n", g_fail);
    return 1;
  }
  printf("host ABI paths OK under the sanitizers (%d launches planned)\n", g_launches);
  return 0;
}
