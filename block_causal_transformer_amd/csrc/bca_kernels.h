// Internal launch interface between the C ABI shim and the HIP kernels.
// Shapes arrive here already validated by the shim.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace bca {

struct AttnDims {
  int op;                 // 0 = space, 1 = time, 2 = time over a KV cache (decode)
  int B, T, N, Hq, Hkv, D;
  int dtype;              // 0 = bf16, 1 = fp32
  int window;             // time: 0 = unbounded causal
  int agent_begin, agent_count;  // space
  float scale;            // softmax scale (> 0)
  // decode only: the T query frames are absolute frames q_frame0 .. ; k and v
  // hold kv_frames frames per slot, absolute frame f at position f % kv_frames
  int kv_frames = 0;
  int q_frame0 = 0;
  // debug: fill the kernels' LDS with NaN bit patterns before staging, so
  // that a read of LDS no thread wrote shows up in the results
  int poison = 0;
  // backward: do not run windowed time attention over more than one key
  // block as segments of the fused kernel (whose fp32 dK, dV partials need
  // more workspace) but as the two-kernel path (Delta workspace only)
  int no_seg = 0;
};

// AttnDims::op of the decode call (the kernels' OP_DECODE).
constexpr int OP_DECODE_ID = 2;

// Key frames a decode call reads: [first, last] in absolute frame indices.
inline void decode_key_range(const AttnDims& d, int& first, int& last) {
  // (T - 1) first: q_frame0 + T - 1 <= INT32_MAX is validated, q_frame0 + T
  // need not fit
  last = d.q_frame0 + (d.T - 1);
  first = (d.window > 0 && d.q_frame0 - d.window + 1 > 0) ? d.q_frame0 - d.window + 1 : 0;
}

// Time attention split into workgroups of `rows_per_wg` folded rows (G per
// position): the largest number of key positions one workgroup can see,
// counting the 32-key alignment of its first key (window W > 0, L frames).
inline int time_wg_key_span(int L, int G, int W, long rows_per_wg) {
  const long rows = (long)L * G;
  int span = 0;
  for (long r0 = 0; r0 < rows; r0 += rows_per_wg) {
    const long r1 = r0 + rows_per_wg < rows ? r0 + rows_per_wg : rows;
    const int p0 = (int)(r0 / G), p1 = (int)((r1 - 1) / G);
    const int k0 = (p0 - W + 1 > 0 ? p0 - W + 1 : 0) & ~31;
    if (p1 + 1 - k0 > span) span = p1 + 1 - k0;
  }
  return span;
}

// Keys per LDS block of the MFMA backward: the dkv kernel gives every such
// block its own workgroup (and forms dQ itself when a problem has only one),
// and the dq kernel streams longer problems through LDS in blocks of this
// many keys.
constexpr int kBwdKeyBlock = 320;

// MFMA kernels: bf16, D = 64.
hipError_t launch_attn_fwd_bf16(const AttnDims& d, const void* q, const void* k, const void* v,
                                void* o, float* lse, hipStream_t stream);
hipError_t launch_attn_bwd_bf16(const AttnDims& d, const void* q, const void* k, const void* v,
                                const void* o, const float* lse, const void* dout, void* dq,
                                void* dk, void* dv, void* workspace, hipStream_t stream);
// Workspace of the MFMA backward: the fp32 Delta = rowsum(dO * O) per
// (query, head), written by its first kernel and read by its second.
size_t bwd_bf16_workspace_bytes(const AttnDims& d);

// Workspace of the fused MFMA backward (one key block per problem) on the
// current device: when its problems fill the CUs in rounds and the last
// round is at most half full, that round's problems run as two workgroups
// each (split by rows) whose fp32 dK, dV partials (2 x keys x 128 floats
// per problem) go here; 0 when nothing is split (or there is no device).
size_t bwd_split_bytes(const AttnDims& d);

// Size of the static device scratch of the no-allocation backward (the
// Delta workspace, one fp32 per (query, head), or the split partials above):
// 64 MiB, i.e. up to 2^24 (query, head) rows per call.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
// Device address of that scratch on the current device (looked up once per
// device with hipGetSymbolAddress and kept); allocates nothing.
hipError_t noalloc_scratch(void** ptr);

// Generic VALU kernels: fp32 or bf16 storage, D = 32 or 64, any length.
hipError_t launch_attn_fwd_generic(const AttnDims& d, const void* q, const void* k,
                                   const void* v, void* o, float* lse, hipStream_t stream);
hipError_t launch_attn_bwd_generic(const AttnDims& d, const void* q, const void* k,
                                   const void* v, const void* o, const float* lse,
                                   const void* dout, void* dq, void* dk, void* dv,
                                   float* delta_ws, hipStream_t stream);

// Projections beside attention: M token rows, d_model features, Hq / Hkv
// heads of width D.
struct ProjDims {
  int64_t M;
  int d_model, Hq, Hkv, D;
};

// RMS norm then the QKV projection: the gain is folded into a bf16 copy of
// the weights in `workspace` (qkv_workspace_bytes: that copy, then M fp32
// rstd values used when `rstd` is NULL), the rows' rstd scales the fp32 sums.
inline size_t qkv_weight_bytes(const ProjDims& d) {
  const size_t b = (size_t)(d.Hq + 2 * d.Hkv) * d.D * d.d_model * 2;
  return (b + 255) & ~(size_t)255;  // rstd starts 256-byte aligned
}
inline size_t qkv_workspace_bytes(const ProjDims& d) { return qkv_weight_bytes(d) + (size_t)d.M * 4; }
hipError_t launch_rmsnorm_qkv(const ProjDims& d, const void* x, const float* gain, float eps,
                              const void* w, void* q, void* k, void* v, float* rstd,
                              void* workspace, hipStream_t stream);
// y = residual (may be NULL) + o w^T.
hipError_t launch_out_proj(const ProjDims& d, const void* o, const void* w, const void* residual,
                           void* y, hipStream_t stream);

// Short problems (bf16, head_dim 64, space or time op with at most 32 key
// positions and at most 64 folded query rows): one wave per problem.
hipError_t launch_attn_fwd_short(const AttnDims& d, const void* q, const void* k, const void* v,
                                 void* o, float* lse, hipStream_t stream);
hipError_t launch_attn_bwd_short(const AttnDims& d, const void* q, const void* k, const void* v,
                                 const void* o, const float* lse, const void* dout, void* dq,
                                 void* dk, void* dv, hipStream_t stream);
inline bool uses_short(const AttnDims& d) {
  if (d.dtype != 0 || d.D != 64 || (d.op != 0 && d.op != 1)) return false;
  const int L = d.op == 0 ? d.N : d.T;
  return L <= 32 && L * (d.Hq / d.Hkv) <= 64;
}

// True when the backward of these dims runs on the MFMA kernels (bf16,
// head_dim 64, any length).
inline bool bwd_uses_mfma(const AttnDims& d) { return d.dtype == 0 && d.D == 64; }

inline bool fwd_uses_mfma(const AttnDims& d) { return d.dtype == 0 && d.D == 64; }

// Positions a problem attends over: tokens (space) or frames (time).
inline int attended_length(const AttnDims& d) { return d.op == 0 ? d.N : d.T; }

// Limits of the MFMA kernels: folded rows r = position * G + head are
// turned back into (position, head) in fp32, exact for G <= 256 and fewer
// than 2^21 rows per problem.
constexpr int kMaxGroup = 256;
constexpr long kMaxFoldedRows = 1L << 21;

// True when the backward needs the Delta workspace: the MFMA path whose
// problems span more than one key block (dQ then comes from a second
// kernel that reads Delta), and the generic VALU path.  (The fused MFMA
// path may still take a workspace for split problems: bwd_split_bytes.)
inline bool bwd_needs_workspace(const AttnDims& d) {
  if (uses_short(d)) return false;
  if (bwd_uses_mfma(d)) return attended_length(d) > kBwdKeyBlock;
  return true;
}

}  // namespace bca
