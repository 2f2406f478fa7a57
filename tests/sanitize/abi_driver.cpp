// Host driver for an AddressSanitizer / UndefinedBehaviorSanitizer build of
// the C ABI shim (block_causal_transformer_amd/csrc/bca_abi.cpp, linked in).
// Test infrastructure.  The kernel launchers and the three HIP runtime calls
// the shim makes are replaced by stubs that record the call, so validation,
// dispatch and error reporting run on the host with no device: every entry
// point is driven with valid descriptors (fake, never dereferenced device
// pointers), with each kind of invalid argument, and with sizes at and past
// every limit (where an integer overflow would show up under UBSan).
// Exit status 0 = all expectations held.
#include <hip/hip_runtime_api.h>
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bca.h"
#include "bca_kernels.h"

static int g_launches = 0, g_syncs = 0;
static bca::AttnDims g_last;

// ---- stubs of the HIP runtime calls the shim makes
extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }
extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }
extern "C" hipError_t hipStreamSynchronize(hipStream_t) {
  ++g_syncs;
  return hipSuccess;
}

// ---- stubs of the kernel launchers
namespace bca {
static hipError_t rec(const AttnDims& d) {
  g_last = d;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_attn_fwd_bf16(const AttnDims& d, const void*, const void*, const void*, void*, float*,
                                hipStream_t) { return rec(d); }
hipError_t launch_attn_bwd_bf16(const AttnDims& d, const void*, const void*, const void*, const void*,
                                const float*, const void*, void*, void*, void*, void*, hipStream_t) {
  return rec(d);
}
size_t bwd_bf16_workspace_bytes(const AttnDims& d) { return (size_t)d.B * d.T * d.N * d.Hq * 4; }
size_t bwd_split_bytes(const AttnDims&) { return 0; }  // no device in this build
hipError_t launch_attn_fwd_generic(const AttnDims& d, const void*, const void*, const void*, void*, float*,
                                   hipStream_t) { return rec(d); }
hipError_t launch_attn_bwd_generic(const AttnDims& d, const void*, const void*, const void*, const void*,
                                   const float*, const void*, void*, void*, void*, float*, hipStream_t) {
  return rec(d);
}
hipError_t launch_attn_fwd_short(const AttnDims& d, const void*, const void*, const void*, void*, float*,
                                 hipStream_t) { return rec(d); }
hipError_t launch_attn_bwd_short(const AttnDims& d, const void*, const void*, const void*, const void*,
                                 const float*, const void*, void*, void*, void*, hipStream_t) {
  return rec(d);
}
hipError_t launch_rmsnorm_qkv(const ProjDims&, const void*, const float*, float, const void*, void*, void*,
                              void*, float*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_out_proj(const ProjDims&, const void*, const void*, const void*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
static int g_lookups = 0;
hipError_t noalloc_scratch(void** ptr) {
  ++g_lookups;
  *ptr = reinterpret_cast<void*>(0x20000);
  return hipSuccess;
}
}  // namespace bca

static int fails = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "FAIL line %d: %s (%s)\n", __LINE__, #cond, bca_last_error()); \
      ++fails;                                                           \
    }                                                                    \
  } while (0)

static void* P = reinterpret_cast<void*>(0x10000);       // aligned, never dereferenced
static void* MIS = reinterpret_cast<void*>(0x10008);

static int fwd(int op, bca_shape s, bca_mask m, void* q = P, void* lse = P) {
  auto f = op == BCA_OP_SPACE ? space_attn_fwd : time_attn_fwd;
  return f(&s, &m, q, P, P, P, static_cast<float*>(lse), nullptr);
}
static int bwd(int op, bca_shape s, bca_mask m, void* ws, size_t wsb, void* dq = P) {
  auto f = op == BCA_OP_SPACE ? space_attn_bwd : time_attn_bwd;
  return f(&s, &m, P, P, P, P, static_cast<const float*>(P), P, dq, P, P, ws, wsb, nullptr);
}

int main() {
  const bca_shape s3 = {4, 64, 290, 30, 3, 64, BCA_BF16};
  const bca_mask ms = {0, 0, 289, 1, 0.f}, mt = {1, 192, 0, 0, 0.f};
  // valid calls reach exactly one launcher each, with the descriptor's values
  int before = g_launches;
  EXPECT(fwd(BCA_OP_SPACE, s3, ms) == BCA_OK);
  EXPECT(g_launches == before + 1 && g_last.N == 290 && g_last.agent_begin == 289 && g_last.window == 0);
  EXPECT(fwd(BCA_OP_TIME, s3, mt) == BCA_OK && g_last.window == 192 && g_last.agent_count == 0);
  EXPECT(bwd(BCA_OP_SPACE, s3, ms, nullptr, 0) == BCA_OK);  // one key block: no workspace
  EXPECT(strcmp(bca_last_error(), "") == 0);
  const bca_shape s5 = {1, 16, 1432, 24, 24, 64, BCA_BF16};
  const size_t need = bca_bwd_workspace_bytes(BCA_OP_SPACE, &s5);
  EXPECT(need == (size_t)16 * 1432 * 24 * 4);
  EXPECT(bwd(BCA_OP_SPACE, s5, {0, 0, 0, 0, 0.f}, nullptr, need) == BCA_ERR_INVALID_ARG);
  EXPECT(bwd(BCA_OP_SPACE, s5, {0, 0, 0, 0, 0.f}, P, need - 1) == BCA_ERR_INVALID_ARG);
  EXPECT(bwd(BCA_OP_SPACE, s5, {0, 0, 0, 0, 0.f}, MIS, need) == BCA_ERR_INVALID_ARG);
  EXPECT(bwd(BCA_OP_SPACE, s5, {0, 0, 0, 0, 0.f}, P, need) == BCA_OK);
  // pointers
  EXPECT(fwd(BCA_OP_SPACE, s3, ms, nullptr) == BCA_ERR_INVALID_ARG);
  EXPECT(fwd(BCA_OP_SPACE, s3, ms, MIS) == BCA_ERR_INVALID_ARG);
  EXPECT(bwd(BCA_OP_TIME, s3, mt, nullptr, 0, MIS) == BCA_ERR_INVALID_ARG);
  EXPECT(space_attn_fwd(nullptr, &ms, P, P, P, P, nullptr, nullptr) == BCA_ERR_INVALID_ARG);
  EXPECT(time_attn_fwd(&s3, nullptr, P, P, P, P, nullptr, nullptr) == BCA_ERR_INVALID_ARG);
  // sizes at and past every limit (no launch may happen for a refused call)
  before = g_launches;
  const int big[] = {0, -1, INT_MIN, INT_MAX};
  for (int v : big) {
    bca_shape s = s3;
    s.B = v;
    EXPECT(fwd(BCA_OP_SPACE, s, ms) != BCA_OK);
    s = s3;
    s.T = v;
    EXPECT(fwd(BCA_OP_TIME, s, mt) != BCA_OK);
    s = s3;
    s.N = v;
    EXPECT(fwd(BCA_OP_SPACE, s, {0, 0, 0, 0, 0.f}) != BCA_OK);
    s = s3;
    s.Hq = v;
    EXPECT(fwd(BCA_OP_SPACE, s, ms) != BCA_OK);
    s = s3;
    s.Hkv = v;
    EXPECT(bwd(BCA_OP_SPACE, s, ms, P, SIZE_MAX) != BCA_OK);
    EXPECT(bca_bwd_workspace_bytes(BCA_OP_TIME, &s) == 0);
  }
  {
    bca_shape s = {INT_MAX, INT_MAX, INT_MAX, INT_MAX, 1, 64, BCA_BF16};
    EXPECT(fwd(BCA_OP_SPACE, s, {0, 0, 0, 0, 0.f}) == BCA_ERR_INVALID_ARG);
    s = {1, 1, 8192, 256, 1, 64, BCA_BF16};
    EXPECT(fwd(BCA_OP_SPACE, s, {0, 0, 0, 0, 0.f}) == BCA_ERR_UNSUPPORTED);
    s = {1, INT_MAX / 2, 1, 256, 1, 64, BCA_BF16};
    EXPECT(fwd(BCA_OP_TIME, s, mt) != BCA_OK);
    s = {1, 1, 16, 257, 1, 64, BCA_BF16};
    EXPECT(fwd(BCA_OP_SPACE, s, {0, 0, 0, 0, 0.f}) == BCA_ERR_UNSUPPORTED);
  }
  EXPECT(fwd(BCA_OP_SPACE, s3, {0, 0, INT_MAX, INT_MAX, 0.f}) == BCA_ERR_INVALID_ARG);
  EXPECT(fwd(BCA_OP_SPACE, s3, {0, 0, INT_MIN, 1, 0.f}) == BCA_ERR_INVALID_ARG);
  EXPECT(fwd(BCA_OP_TIME, s3, {1, INT_MIN, 0, 0, 0.f}) == BCA_ERR_INVALID_ARG);
  EXPECT(fwd(BCA_OP_TIME, s3, {1, INT_MAX, 0, 0, 0.f}) == BCA_OK);  // a window past T is unbounded
  EXPECT(g_launches == before + 1);
  // decode: ring sizes and frame indices at their limits
  {
    bca_shape s = {1, 1, 290, 30, 3, 64, BCA_BF16};
    EXPECT(time_attn_decode_fwd(&s, &mt, P, P, P, 192, 1000, P, static_cast<float*>(P), nullptr) == BCA_OK);
    EXPECT(g_last.op == bca::OP_DECODE_ID && g_last.q_frame0 == 1000 && g_last.kv_frames == 192);
    EXPECT(time_attn_decode_fwd(&s, &mt, P, P, P, 191, 1000, P, static_cast<float*>(P), nullptr) ==
           BCA_ERR_INVALID_ARG);
    EXPECT(time_attn_decode_fwd(&s, &mt, P, P, P, INT_MAX, INT_MAX, P, static_cast<float*>(P), nullptr) ==
           BCA_OK);
    s.T = 2;
    EXPECT(time_attn_decode_fwd(&s, &mt, P, P, P, INT_MAX, INT_MAX, P, static_cast<float*>(P), nullptr) ==
           BCA_ERR_INVALID_ARG);
    EXPECT(time_attn_decode_fwd(&s, &mt, P, P, P, INT_MIN, 5, P, static_cast<float*>(P), nullptr) ==
           BCA_ERR_INVALID_ARG);
    const bca_mask m0 = {1, 0, 0, 0, 0.f};
    s = {1, 1, 4, 256, 1, 64, BCA_BF16};
    EXPECT(time_attn_decode_fwd(&s, &m0, P, P, P, 9000, 8191, P, static_cast<float*>(P), nullptr) ==
           BCA_ERR_UNSUPPORTED);
  }
  // projections
  {
    bca_proj_shape ps = {74240, 1920, 30, 3, 64};
    const size_t w = bca_qkv_workspace_bytes(&ps);
    EXPECT(w == ((size_t)2304 * 1920 * 2 + 255) / 256 * 256 + (size_t)74240 * 4);  // folded weights, rstd
    EXPECT(rmsnorm_qkv_fwd(&ps, P, static_cast<float*>(P), 1e-6f, P, P, P, P, nullptr, P, w, nullptr) == BCA_OK);
    EXPECT(rmsnorm_qkv_fwd(&ps, P, static_cast<float*>(P), -1.f, P, P, P, P, nullptr, P, w, nullptr) ==
           BCA_ERR_INVALID_ARG);
    EXPECT(out_proj_fwd(&ps, P, P, nullptr, P, nullptr) == BCA_OK);
    const int64_t bigm[] = {0, -1, INT64_MAX, (int64_t)1 << 40};
    for (int64_t m : bigm) {
      bca_proj_shape b = ps;
      b.M = m;
      EXPECT(out_proj_fwd(&b, P, P, nullptr, P, nullptr) != BCA_OK);
      EXPECT(bca_qkv_workspace_bytes(&b) == 0);
    }
    bca_proj_shape b = {1, INT_MAX - 7, INT_MAX, INT_MAX, INT_MAX - 7};
    EXPECT(out_proj_fwd(&b, P, P, nullptr, P, nullptr) != BCA_OK);
  }
  // the no-allocation backward: scratch only when the shape needs a workspace,
  // refused past the static array's size
  {
    const bca_shape sl = {1, 1024, 290, 30, 3, 64, BCA_BF16};  // 35.6 MB of Delta
    before = g_launches;
    EXPECT(time_attn_bwd_noalloc(&sl, &mt, P, P, P, P, static_cast<float*>(P), P, P, P, P, nullptr) == BCA_OK);
    EXPECT(g_launches == before + 1 && bca::g_lookups == 1);
    EXPECT(time_attn_bwd_noalloc(&s3, &mt, P, P, P, P, static_cast<float*>(P), P, P, P, P, nullptr) == BCA_OK);
    EXPECT(bca::g_lookups == 1);  // 256 frames: one key block, no workspace
    const bca_shape sh = {1, 1024, 1000, 30, 3, 64, BCA_BF16};  // 123 MB of Delta
    EXPECT(time_attn_bwd_noalloc(&sh, &mt, P, P, P, P, static_cast<float*>(P), P, P, P, P, nullptr) ==
           BCA_ERR_INVALID_ARG);
    EXPECT(strstr(bca_last_error(), "static scratch") != nullptr);
    EXPECT(time_attn_bwd_noalloc(&sl, &mt, P, nullptr, P, P, static_cast<float*>(P), P, P, P, P, nullptr) ==
           BCA_ERR_INVALID_ARG);
    EXPECT(time_attn_bwd_noalloc(&sl, &ms, P, P, P, P, static_cast<float*>(P), P, P, P, P, nullptr) ==
           BCA_ERR_UNSUPPORTED);
  }
  // BCA_SYNC synchronizes after a launch; status strings
  setenv("BCA_SYNC", "1", 1);
  const int syncs = g_syncs;
  EXPECT(fwd(BCA_OP_SPACE, s3, ms) == BCA_OK && g_syncs == syncs + 1);
  unsetenv("BCA_SYNC");
  setenv("BCA_DEBUG_LDS_POISON", "1", 1);
  EXPECT(fwd(BCA_OP_SPACE, s3, ms) == BCA_OK && g_last.poison == 1);
  unsetenv("BCA_DEBUG_LDS_POISON");
  EXPECT(fwd(BCA_OP_SPACE, s3, ms) == BCA_OK && g_last.poison == 0);
  EXPECT(strcmp(bca_status_string(BCA_ERR_HIP), "BCA_ERR_HIP") == 0);
  EXPECT(strcmp(bca_status_string(-5), "BCA_UNKNOWN_STATUS") == 0);
  EXPECT(bca_abi_version() == BCA_ABI_VERSION);
  if (fails) return 1;
  printf("abi sanitizer driver: ok\n");
  return 0;
}
