// C ABI shim: host-side validation, kernel selection and error reporting for
// the declarations in include/bca.h.  Validation is synchronous, touches no
// device memory and happens before any launch.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "bca.h"
#include "bca_kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Fills `d` from the descriptors; returns BCA_OK or an error status.
int validate(int op, const bca_shape* s, const bca_mask* m, bca::AttnDims* d) {
  if (!s || !m) return fail(BCA_ERR_INVALID_ARG, "shape or mask descriptor is NULL");
  if (s->B <= 0 || s->T <= 0 || s->N <= 0 || s->Hq <= 0 || s->Hkv <= 0 || s->D <= 0)
    return fail(BCA_ERR_INVALID_ARG, "non-positive size (B=%d T=%d N=%d Hq=%d Hkv=%d D=%d)",
                s->B, s->T, s->N, s->Hq, s->Hkv, s->D);
  if (s->Hq % s->Hkv != 0)
    return fail(BCA_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", s->Hq, s->Hkv);
  if (s->dtype != BCA_BF16 && s->dtype != BCA_F32)
    return fail(BCA_ERR_UNSUPPORTED, "unknown dtype %d", s->dtype);
  if (s->D != 32 && s->D != 64) return fail(BCA_ERR_UNSUPPORTED, "head_dim %d (need 32 or 64)", s->D);
  // element counts must fit the kernels' 64-bit offsets and 32-bit grids
  const double elems = (double)s->B * s->T * s->N * s->Hq * s->D;
  if (elems > 4.0e15) return fail(BCA_ERR_INVALID_ARG, "tensor too large (%.3g elements)", elems);
  const double rows = (double)s->B * s->T * s->N * s->Hq;
  if (rows / 128.0 > 2.0e9) return fail(BCA_ERR_INVALID_ARG, "too many rows for the launch grid");
  if (m->agent_begin < 0 || m->agent_count < 0 ||
      (int64_t)m->agent_begin + m->agent_count > s->N)
    return fail(BCA_ERR_INVALID_ARG, "agent range [%d, %d+%d) not inside [0, N=%d]",
                m->agent_begin, m->agent_begin, m->agent_count, s->N);
  if (m->window < 0) return fail(BCA_ERR_INVALID_ARG, "window %d < 0", m->window);
  if (!(isfinite(m->softmax_scale))) return fail(BCA_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (op == BCA_OP_SPACE) {
    if (m->causal != 0) return fail(BCA_ERR_UNSUPPORTED, "space attention is not causal (causal=%d)", m->causal);
    if (m->window != 0) return fail(BCA_ERR_UNSUPPORTED, "space attention takes no window (window=%d)", m->window);
  } else {
    if (m->causal != 1) return fail(BCA_ERR_UNSUPPORTED, "time attention must be causal (causal=%d)", m->causal);
  }
  // the kernels fold the G query heads of a KV head into rows
  // position * G + head of one problem
  const int G = s->Hq / s->Hkv;
  if (G > bca::kMaxGroup)
    return fail(BCA_ERR_UNSUPPORTED, "%d query heads per KV head (at most %d)", G, bca::kMaxGroup);
  const long L = op == BCA_OP_SPACE ? s->N : s->T;
  if (L * G >= bca::kMaxFoldedRows)
    return fail(BCA_ERR_UNSUPPORTED, "%ld positions x %d heads per KV head is %ld rows per problem "
                "(fewer than %ld supported)", L, G, L * G, bca::kMaxFoldedRows);
  d->op = op;
  d->B = s->B;
  d->T = s->T;
  d->N = s->N;
  d->Hq = s->Hq;
  d->Hkv = s->Hkv;
  d->D = s->D;
  d->dtype = s->dtype;
  d->window = op == BCA_OP_TIME ? m->window : 0;
  d->agent_begin = op == BCA_OP_SPACE ? m->agent_begin : 0;
  d->agent_count = op == BCA_OP_SPACE ? m->agent_count : 0;
  d->scale = m->softmax_scale > 0.f ? m->softmax_scale : 1.0f / sqrtf((float)s->D);
  return BCA_OK;
}

int check_ptrs(const char* const* names, const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i]) return fail(BCA_ERR_INVALID_ARG, "pointer '%s' is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(BCA_ERR_INVALID_ARG, "pointer '%s' is not 16-byte aligned", names[i]);
  }
  return BCA_OK;
}

size_t workspace_bytes(const bca::AttnDims& d) {
  if (bca::uses_short(d)) return 0;
  if (!bca::bwd_needs_workspace(d)) return bca::bwd_uses_mfma(d) ? bca::bwd_split_bytes(d) : 0;
  if (bca::bwd_uses_mfma(d)) return bca::bwd_bf16_workspace_bytes(d);
  return (size_t)d.B * d.T * d.N * d.Hq * sizeof(float);
}

// Debug switches, read from the environment at every call:
//  BCA_SYNC=1               synchronize the stream after every launch and
//                           report a kernel fault as BCA_ERR_HIP from the call
//  BCA_DEBUG_LDS_POISON=1   fill the attention kernels' LDS with NaN bit
//                           patterns before staging (a read of LDS that no
//                           thread wrote then shows up in the results)
bool env_flag(const char* name) {
  const char* v = getenv(name);
  return v && v[0] && strcmp(v, "0") != 0;
}
bool sync_after_launch() { return env_flag("BCA_SYNC"); }
int lds_poison() { return env_flag("BCA_DEBUG_LDS_POISON") ? 1 : 0; }

// Clears an error an earlier, unrelated HIP call may have left in this
// thread's error state, so that the check after the launch reports only the
// launch's own.
void clear_stale_hip_error() { (void)hipGetLastError(); }

int hip_status(hipError_t e, const char* what, void* stream) {
  if (e == hipSuccess && sync_after_launch()) {
    e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(BCA_ERR_HIP, "%s (BCA_SYNC): %s", what, hipGetErrorString(e));
  }
  if (e == hipSuccess) return BCA_OK;
  return fail(BCA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int do_fwd(int op, const bca_shape* shape, const bca_mask* mask, const void* q, const void* k,
           const void* v, void* o, float* lse, void* stream) {
  bca::AttnDims d;
  int st = validate(op, shape, mask, &d);
  if (st) return st;
  const char* names[] = {"q", "k", "v", "o", "lse"};
  const void* ptrs[] = {q, k, v, o, lse};
  st = check_ptrs(names, ptrs, 5);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  d.poison = lds_poison();
  clear_stale_hip_error();
  hipError_t e = bca::uses_short(d)      ? bca::launch_attn_fwd_short(d, q, k, v, o, lse, s)
                  : bca::fwd_uses_mfma(d) ? bca::launch_attn_fwd_bf16(d, q, k, v, o, lse, s)
                                          : bca::launch_attn_fwd_generic(d, q, k, v, o, lse, s);
  st = hip_status(e, op == BCA_OP_SPACE ? "space_attn_fwd launch" : "time_attn_fwd launch", stream);
  if (st == BCA_OK) g_last_error.clear();
  return st;
}

int do_bwd(int op, const bca_shape* shape, const bca_mask* mask, const void* q, const void* k,
           const void* v, const void* o, const float* lse, const void* dout, void* dq, void* dk,
           void* dv, void* workspace, size_t ws_bytes, void* stream, bool segments = true) {
  bca::AttnDims d;
  int st = validate(op, shape, mask, &d);
  if (st) return st;
  d.no_seg = segments ? 0 : 1;
  const char* names[] = {"q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv"};
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  st = check_ptrs(names, ptrs, 9);
  if (st) return st;
  const size_t need = workspace_bytes(d);
  if (need > 0) {
    if (ws_bytes < need)
      return fail(BCA_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu required",
                  ws_bytes, need);
    if (!workspace || !aligned16(workspace))
      return fail(BCA_ERR_INVALID_ARG, "workspace is NULL or not 16-byte aligned");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  d.poison = lds_poison();
  clear_stale_hip_error();
  // the short kernels form Delta per row themselves and leave the workspace alone
  hipError_t e = bca::uses_short(d)
                     ? bca::launch_attn_bwd_short(d, q, k, v, o, lse, dout, dq, dk, dv, s)
                 : bca::bwd_uses_mfma(d)
                     ? bca::launch_attn_bwd_bf16(d, q, k, v, o, lse, dout, dq, dk, dv, workspace, s)
                     : bca::launch_attn_bwd_generic(d, q, k, v, o, lse, dout, dq, dk, dv,
                                                    static_cast<float*>(workspace), s);
  st = hip_status(e, op == BCA_OP_SPACE ? "space_attn_bwd launch" : "time_attn_bwd launch", stream);
  if (st == BCA_OK) g_last_error.clear();
  return st;
}

// The backward with its workspace taken from the library's static device
// scratch: allocates nothing (no hipMalloc, no library allocation).
int do_bwd_noalloc(int op, const bca_shape* shape, const bca_mask* mask, const void* q,
                   const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, void* stream) {
  bca::AttnDims d;
  int st = validate(op, shape, mask, &d);
  if (st) return st;
  const char* names[] = {"q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv"};
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  st = check_ptrs(names, ptrs, 9);
  if (st) return st;
  // windowed time attention over more than one key block runs as segments
  // whose dK, dV partials need more workspace than the Delta rows of the
  // two-kernel path; when they do not fit the scratch, the latter is used
  size_t need = workspace_bytes(d);
  bool segments = true;
  if (need > bca::kNoAllocScratchBytes) {
    d.no_seg = 1;
    need = workspace_bytes(d);
    segments = false;
  }
  if (need > bca::kNoAllocScratchBytes)
    return fail(BCA_ERR_INVALID_ARG,
                "this shape needs %zu bytes of workspace; the static scratch holds %zu "
                "(at most %zu query-head rows)", need, bca::kNoAllocScratchBytes,
                bca::kNoAllocScratchBytes / sizeof(float));
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = bca::noalloc_scratch(&ws);
    if (e != hipSuccess)
      return fail(BCA_ERR_HIP, "static scratch lookup: %s", hipGetErrorString(e));
  }
  return do_bwd(op, shape, mask, q, k, v, o, lse, dout, dq, dk, dv, ws, need, stream, segments);
}

int do_decode_fwd(const bca_shape* shape, const bca_mask* mask, const void* q, const void* kc,
                  const void* vc, int32_t cache_frames, int32_t q_frame0, void* o, float* lse,
                  void* stream) {
  bca::AttnDims d;
  int st = validate(BCA_OP_TIME, shape, mask, &d);
  if (st) return st;
  const char* names[] = {"q", "k_cache", "v_cache", "o", "lse"};
  const void* ptrs[] = {q, kc, vc, o, lse};
  st = check_ptrs(names, ptrs, 5);
  if (st) return st;
  if (cache_frames <= 0) return fail(BCA_ERR_INVALID_ARG, "cache_frames %d <= 0", cache_frames);
  if (q_frame0 < 0) return fail(BCA_ERR_INVALID_ARG, "q_frame0 %d < 0", q_frame0);
  if ((int64_t)q_frame0 + shape->T - 1 > INT32_MAX)
    return fail(BCA_ERR_INVALID_ARG, "q_frame0 + T overflows the frame index");
  if ((double)shape->B * cache_frames * shape->N * shape->Hkv * shape->D > 4.0e15)
    return fail(BCA_ERR_INVALID_ARG, "cache too large");
  d.op = bca::OP_DECODE_ID;
  d.kv_frames = cache_frames;
  d.q_frame0 = q_frame0;
  int first, last;
  bca::decode_key_range(d, first, last);
  if (last - first + 1 > cache_frames)
    return fail(BCA_ERR_INVALID_ARG,
                "a cache of %d frames cannot hold the %d frames [%d, %d] the queries read",
                cache_frames, last - first + 1, first, last);
  if ((long)(last - first + 1) * (d.Hq / d.Hkv) >= bca::kMaxFoldedRows)
    return fail(BCA_ERR_UNSUPPORTED, "the %d frames read x %d heads per KV head exceed the "
                "kernels' %ld rows per problem", last - first + 1, d.Hq / d.Hkv, bca::kMaxFoldedRows);
  hipStream_t s = static_cast<hipStream_t>(stream);
  d.poison = lds_poison();
  clear_stale_hip_error();
  hipError_t e = bca::fwd_uses_mfma(d) ? bca::launch_attn_fwd_bf16(d, q, kc, vc, o, lse, s)
                                       : bca::launch_attn_fwd_generic(d, q, kc, vc, o, lse, s);
  st = hip_status(e, "time_attn_decode_fwd launch", stream);
  if (st == BCA_OK) g_last_error.clear();
  return st;
}

int validate_proj(const bca_proj_shape* s, bca::ProjDims* d) {
  if (!s) return fail(BCA_ERR_INVALID_ARG, "projection shape descriptor is NULL");
  if (s->M <= 0 || s->d_model <= 0 || s->Hq <= 0 || s->Hkv <= 0 || s->D <= 0)
    return fail(BCA_ERR_INVALID_ARG, "non-positive size (M=%lld d_model=%d Hq=%d Hkv=%d D=%d)",
                (long long)s->M, s->d_model, s->Hq, s->Hkv, s->D);
  if (s->d_model % 8 != 0 || s->D % 8 != 0)
    return fail(BCA_ERR_UNSUPPORTED, "d_model (%d) and D (%d) must be multiples of 8", s->d_model, s->D);
  // sizes in double first: (Hq + 2 Hkv) * D overflows 64-bit integers for
  // the largest int32 fields
  const double nout = ((double)s->Hq + 2.0 * s->Hkv) * s->D;
  const double widest = nout > s->d_model ? nout : s->d_model;
  if (nout > (double)(1 << 30) || (double)s->M * widest > 4.0e15 ||
      ((double)s->M / 128.0 + 1.0) * (nout / 128.0 + 1.0) > 2147483647.0)
    return fail(BCA_ERR_INVALID_ARG, "projection too large");
  d->M = s->M;
  d->d_model = s->d_model;
  d->Hq = s->Hq;
  d->Hkv = s->Hkv;
  d->D = s->D;
  return BCA_OK;
}

}  // namespace

extern "C" {

size_t bca_qkv_workspace_bytes(const bca_proj_shape* shape) {
  bca::ProjDims d;
  const std::string saved = g_last_error;
  if (validate_proj(shape, &d) != BCA_OK) {
    g_last_error = saved;
    return 0;
  }
  return bca::qkv_workspace_bytes(d);
}

int rmsnorm_qkv_fwd(const bca_proj_shape* shape, const void* x, const float* gain, float eps,
                    const void* w_qkv, void* q, void* k, void* v, float* rstd, void* workspace,
                    size_t workspace_bytes, void* stream) {
  bca::ProjDims d;
  int st = validate_proj(shape, &d);
  if (st) return st;
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(BCA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const char* names[] = {"x", "gain", "w_qkv", "q", "k", "v", "workspace"};
  const void* ptrs[] = {x, gain, w_qkv, q, k, v, workspace};
  st = check_ptrs(names, ptrs, 7);
  if (st) return st;
  if (rstd && !aligned16(rstd)) return fail(BCA_ERR_INVALID_ARG, "pointer 'rstd' is not 16-byte aligned");
  const size_t need = bca::qkv_workspace_bytes(d);
  if (workspace_bytes < need)
    return fail(BCA_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu required",
                workspace_bytes, need);
  clear_stale_hip_error();
  hipError_t e = bca::launch_rmsnorm_qkv(d, x, gain, eps, w_qkv, q, k, v, rstd, workspace,
                                         static_cast<hipStream_t>(stream));
  st = hip_status(e, "rmsnorm_qkv_fwd launch", stream);
  if (st == BCA_OK) g_last_error.clear();
  return st;
}

int out_proj_fwd(const bca_proj_shape* shape, const void* o, const void* w_o, const void* residual,
                 void* y, void* stream) {
  bca::ProjDims d;
  int st = validate_proj(shape, &d);
  if (st) return st;
  const char* names[] = {"o", "w_o", "y"};
  const void* ptrs[] = {o, w_o, y};
  st = check_ptrs(names, ptrs, 3);
  if (st) return st;
  if (residual && !aligned16(residual))
    return fail(BCA_ERR_INVALID_ARG, "pointer 'residual' is not 16-byte aligned");
  clear_stale_hip_error();
  hipError_t e = bca::launch_out_proj(d, o, w_o, residual, y, static_cast<hipStream_t>(stream));
  st = hip_status(e, "out_proj_fwd launch", stream);
  if (st == BCA_OK) g_last_error.clear();
  return st;
}

int time_attn_decode_fwd(const bca_shape* shape, const bca_mask* mask, const void* q,
                         const void* k_cache, const void* v_cache, int32_t cache_frames,
                         int32_t q_frame0, void* o, float* lse, void* stream) {
  return do_decode_fwd(shape, mask, q, k_cache, v_cache, cache_frames, q_frame0, o, lse, stream);
}

int space_attn_fwd(const bca_shape* shape, const bca_mask* mask, const void* q, const void* k,
                   const void* v, void* o, float* lse, void* stream) {
  return do_fwd(BCA_OP_SPACE, shape, mask, q, k, v, o, lse, stream);
}

int time_attn_fwd(const bca_shape* shape, const bca_mask* mask, const void* q, const void* k,
                  const void* v, void* o, float* lse, void* stream) {
  return do_fwd(BCA_OP_TIME, shape, mask, q, k, v, o, lse, stream);
}

int space_attn_bwd(const bca_shape* shape, const bca_mask* mask, const void* q, const void* k,
                   const void* v, const void* o, const float* lse, const void* dout, void* dq,
                   void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  return do_bwd(BCA_OP_SPACE, shape, mask, q, k, v, o, lse, dout, dq, dk, dv, workspace,
                workspace_bytes, stream);
}

int time_attn_bwd(const bca_shape* shape, const bca_mask* mask, const void* q, const void* k,
                  const void* v, const void* o, const float* lse, const void* dout, void* dq,
                  void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  return do_bwd(BCA_OP_TIME, shape, mask, q, k, v, o, lse, dout, dq, dk, dv, workspace,
                workspace_bytes, stream);
}

int time_attn_bwd_noalloc(const bca_shape* shape, const bca_mask* mask, const void* q,
                          const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, void* stream) {
  return do_bwd_noalloc(BCA_OP_TIME, shape, mask, q, k, v, o, lse, dout, dq, dk, dv, stream);
}

size_t bca_bwd_workspace_bytes(int op, const bca_shape* shape) {
  if (op != BCA_OP_SPACE && op != BCA_OP_TIME) return 0;
  bca_mask m;
  m.causal = op == BCA_OP_TIME ? 1 : 0;
  m.window = 0;
  m.agent_begin = 0;
  m.agent_count = 0;
  m.softmax_scale = 0.f;
  bca::AttnDims d;
  const std::string saved = g_last_error;
  if (validate(op, shape, &m, &d) != BCA_OK) {
    g_last_error = saved;
    return 0;
  }
  size_t need = workspace_bytes(d);
  // the need depends on the time op's window, which the query does not
  // take: the largest over all windows.  Windowed time attention over more
  // than one key block runs as segments of at least 128 positions, whose
  // partials take the most room at exactly 128 (window 193).
  if (op == BCA_OP_TIME) {
    d.window = 193;
    need = std::max(need, workspace_bytes(d));
  }
  return need;
}

const char* bca_status_string(int status) {
  switch (status) {
    case BCA_OK: return "BCA_OK";
    case BCA_ERR_INVALID_ARG: return "BCA_ERR_INVALID_ARG";
    case BCA_ERR_UNSUPPORTED: return "BCA_ERR_UNSUPPORTED";
    case BCA_ERR_HIP: return "BCA_ERR_HIP";
    default: return "BCA_UNKNOWN_STATUS";
  }
}

const char* bca_last_error(void) { return g_last_error.c_str(); }

int bca_abi_version(void) { return BCA_ABI_VERSION; }

}  // extern "C"
