// Generic VALU kernels for space and time attention: fp32 or bf16 storage,
// head_dim 32 or 64, any sequence length.  They serve the fp32 path (whose
// tolerance calls for plain fp32 arithmetic, not bf16 MFMA operands), bf16 at
// head_dim 32, and the backward of problems longer than the MFMA backward's
// LDS-resident limit.  All arithmetic is fp32.
//
// Same definition as the MFMA kernels (Open Dreamer articles,
// pro.edgex.exchange fr-FR edition, sections "Architecture" and
// "Configuration d'entraînement"): space attention inside one block with
// world tokens unable to read agent tokens, causal sliding-window time
// attention per token slot, GQA head h -> KV head h / (Hq / Hkv).
//
// Forward: one thread per (unit, position, query head), two passes over the
// visible keys (exact max, then sum and weighted values).  Backward: one
// thread per (unit, position, query head) for Delta and dQ, then one thread
// per (unit, key position, KV head) for dK and dV, so every sum is owned by a
// single thread (deterministic, no atomics).
#include "bca_device.h"
#include "bca_kernels.h"

namespace bca {

namespace {

struct GenParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* out0;  // o (fwd) or dq (bwd)
  void* out1;  // dk
  void* out2;  // dv
  float* lse_out;
  float* delta;
  int op, T, N, Hq, Hkv, G, L, units;
  int window, agent_begin, agent_count;
  float scale;
  // forward of the decode op: Lq query positions, each at key position
  // a + qoff; key position b is absolute frame kfirst + b, stored at frame
  // (kfirst + b) % Tk of k and v.  Plain ops: Lq = L, qoff = kfirst = 0,
  // Tk = T.
  int Lq, qoff, kfirst, Tk;
};

template <typename E>
__device__ __forceinline__ float ldf(const E* p, int64_t i) {
  return (float)p[i];
}

template <typename E>
__device__ __forceinline__ void stf(E* p, int64_t i, float x) {
  p[i] = (E)x;
}

template <typename E, int D>
__global__ __launch_bounds__(128) void gen_fwd_kernel(GenParams p) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.units * p.Lq * p.Hq;
  if (gid >= total) return;
  const int h = (int)(gid % p.Hq);
  const int a = (int)((gid / p.Hq) % p.Lq);
  const int u = (int)(gid / ((int64_t)p.Hq * p.Lq));
  const int g = h / p.G;
  const int mop = p.op == OP_DECODE ? OP_TIME : p.op;
  const UnitGeom gq = unit_geom(mop, u, p.T, p.N, p.Hq, D);
  const UnitGeom gk = unit_geom(mop, u, p.Tk, p.N, p.Hkv, D);
  const UnitGeom gl = unit_geom(mop, u, p.T, p.N, p.Hq, 1);
  const MaskDesc md{mop, p.L, p.window, p.agent_begin, p.agent_count};
  const int ak = a + p.qoff;  // query position among the keys
  const E* q = static_cast<const E*>(p.q) + gq.base + (int64_t)a * gq.pos_stride + (int64_t)h * D;
  const E* k = static_cast<const E*>(p.k) + gk.base + (int64_t)g * D;
  const E* v = static_cast<const E*>(p.v) + gk.base + (int64_t)g * D;
  auto kpos = [&](int b) -> int64_t {
    return (int64_t)(p.op == OP_DECODE ? (p.kfirst + b) % p.Tk : b) * gk.pos_stride;
  };
  float qr[D];
#pragma unroll
  for (int d = 0; d < D; ++d) qr[d] = ldf(q, d);
  float m = -INFINITY;
  for (int b = 0; b < p.L; ++b) {
    if (!visible(md, ak, b)) continue;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = __builtin_fmaf(qr[d], ldf(k + kpos(b), d), s);
    m = fmaxf(m, s * p.scale);
  }
  float l = 0.f;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  for (int b = 0; b < p.L; ++b) {
    if (!visible(md, ak, b)) continue;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = __builtin_fmaf(qr[d], ldf(k + kpos(b), d), s);
    const float e = expf(s * p.scale - m);
    l += e;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(e, ldf(v + kpos(b), d), acc[d]);
  }
  E* o = static_cast<E*>(p.out0) + gq.base + (int64_t)a * gq.pos_stride + (int64_t)h * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) stf(o, d, acc[d] * inv);
  p.lse_out[gl.base + (int64_t)a * gl.pos_stride + h] = m + logf(l);
}

template <typename E, int D>
__global__ __launch_bounds__(128) void gen_bwd_dq_kernel(GenParams p) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.units * p.L * p.Hq;
  if (gid >= total) return;
  const int h = (int)(gid % p.Hq);
  const int a = (int)((gid / p.Hq) % p.L);
  const int u = (int)(gid / ((int64_t)p.Hq * p.L));
  const int g = h / p.G;
  const UnitGeom gq = unit_geom(p.op, u, p.T, p.N, p.Hq, D);
  const UnitGeom gk = unit_geom(p.op, u, p.T, p.N, p.Hkv, D);
  const UnitGeom gl = unit_geom(p.op, u, p.T, p.N, p.Hq, 1);
  const MaskDesc md{p.op, p.L, p.window, p.agent_begin, p.agent_count};
  const int64_t qo = gq.base + (int64_t)a * gq.pos_stride + (int64_t)h * D;
  const E* q = static_cast<const E*>(p.q) + qo;
  const E* o = static_cast<const E*>(p.o) + qo;
  const E* dout = static_cast<const E*>(p.dout) + qo;
  const E* k = static_cast<const E*>(p.k) + gk.base + (int64_t)g * D;
  const E* v = static_cast<const E*>(p.v) + gk.base + (int64_t)g * D;
  float qr[D], dr[D], dq[D];
  float delta = 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = ldf(q, d);
    dr[d] = ldf(dout, d);
    delta = __builtin_fmaf(dr[d], ldf(o, d), delta);
    dq[d] = 0.f;
  }
  const int64_t li = gl.base + (int64_t)a * gl.pos_stride + h;
  const float lse = p.lse[li];
  p.delta[li] = delta;
  for (int b = 0; b < p.L; ++b) {
    if (!visible(md, a, b)) continue;
    const E* kb = k + (int64_t)b * gk.pos_stride;
    const E* vb = v + (int64_t)b * gk.pos_stride;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      s = __builtin_fmaf(qr[d], ldf(kb, d), s);
      dp = __builtin_fmaf(dr[d], ldf(vb, d), dp);
    }
    const float pr = expf(s * p.scale - lse);
    const float ds = pr * (dp - delta) * p.scale;
#pragma unroll
    for (int d = 0; d < D; ++d) dq[d] = __builtin_fmaf(ds, ldf(kb, d), dq[d]);
  }
  E* out = static_cast<E*>(p.out0) + qo;
#pragma unroll
  for (int d = 0; d < D; ++d) stf(out, d, dq[d]);
}

template <typename E, int D>
__global__ __launch_bounds__(128) void gen_bwd_dkv_kernel(GenParams p) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.units * p.L * p.Hkv;
  if (gid >= total) return;
  const int g = (int)(gid % p.Hkv);
  const int b = (int)((gid / p.Hkv) % p.L);
  const int u = (int)(gid / ((int64_t)p.Hkv * p.L));
  const UnitGeom gq = unit_geom(p.op, u, p.T, p.N, p.Hq, D);
  const UnitGeom gk = unit_geom(p.op, u, p.T, p.N, p.Hkv, D);
  const UnitGeom gl = unit_geom(p.op, u, p.T, p.N, p.Hq, 1);
  const MaskDesc md{p.op, p.L, p.window, p.agent_begin, p.agent_count};
  const int64_t ko = gk.base + (int64_t)b * gk.pos_stride + (int64_t)g * D;
  const E* kb = static_cast<const E*>(p.k) + ko;
  const E* vb = static_cast<const E*>(p.v) + ko;
  float kr[D], vr[D], dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    kr[d] = ldf(kb, d);
    vr[d] = ldf(vb, d);
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  for (int h = g * p.G; h < (g + 1) * p.G; ++h) {
    for (int a = 0; a < p.L; ++a) {
      if (!visible(md, a, b)) continue;
      const int64_t qo = gq.base + (int64_t)a * gq.pos_stride + (int64_t)h * D;
      const E* q = static_cast<const E*>(p.q) + qo;
      const E* dout = static_cast<const E*>(p.dout) + qo;
      const int64_t li = gl.base + (int64_t)a * gl.pos_stride + h;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = __builtin_fmaf(ldf(q, d), kr[d], s);
        dp = __builtin_fmaf(ldf(dout, d), vr[d], dp);
      }
      const float pr = expf(s * p.scale - p.lse[li]);
      const float ds = pr * (dp - p.delta[li]) * p.scale;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        dk[d] = __builtin_fmaf(ds, ldf(q, d), dk[d]);
        dv[d] = __builtin_fmaf(pr, ldf(dout, d), dv[d]);
      }
    }
  }
  E* dko = static_cast<E*>(p.out1) + ko;
  E* dvo = static_cast<E*>(p.out2) + ko;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    stf(dko, d, dk[d]);
    stf(dvo, d, dv[d]);
  }
}

GenParams make_params(const AttnDims& d) {
  GenParams p{};
  p.op = d.op;
  p.T = d.T;
  p.N = d.N;
  p.Hq = d.Hq;
  p.Hkv = d.Hkv;
  p.G = d.Hq / d.Hkv;
  p.L = d.op == OP_SPACE ? d.N : d.T;
  p.units = d.op == OP_SPACE ? d.B * d.T : d.B * d.N;
  p.window = d.window;
  p.agent_begin = d.agent_begin;
  p.agent_count = d.agent_count;
  p.scale = d.scale;
  p.Lq = p.L;
  p.qoff = 0;
  p.kfirst = 0;
  p.Tk = d.T;
  if (d.op == OP_DECODE) {
    int first, last;
    decode_key_range(d, first, last);
    p.L = last - first + 1;
    p.Lq = d.T;
    p.qoff = d.q_frame0 - first;
    p.kfirst = first;
    p.Tk = d.kv_frames;
  }
  return p;
}

template <typename E, int D>
hipError_t run_fwd(GenParams p, hipStream_t s) {
  const int64_t total = (int64_t)p.units * p.Lq * p.Hq;
  const int64_t blocks = (total + 127) / 128;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gen_fwd_kernel<E, D>), dim3((unsigned)blocks), dim3(128), 0, s, p);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t run_bwd(GenParams p, hipStream_t s) {
  const int64_t t0 = (int64_t)p.units * p.L * p.Hq;
  const int64_t t1 = (int64_t)p.units * p.L * p.Hkv;
  const int64_t b0 = (t0 + 127) / 128, b1 = (t1 + 127) / 128;
  if (b0 > 0x7fffffff || b1 > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gen_bwd_dq_kernel<E, D>), dim3((unsigned)b0), dim3(128), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gen_bwd_dkv_kernel<E, D>), dim3((unsigned)b1), dim3(128), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_generic(const AttnDims& d, const void* q, const void* k,
                                   const void* v, void* o, float* lse, hipStream_t stream) {
  GenParams p = make_params(d);
  p.q = q;
  p.k = k;
  p.v = v;
  p.out0 = o;
  p.lse_out = lse;
  if (d.dtype == 1) return d.D == 32 ? run_fwd<float, 32>(p, stream) : run_fwd<float, 64>(p, stream);
  return d.D == 32 ? run_fwd<bf16, 32>(p, stream) : run_fwd<bf16, 64>(p, stream);
}

hipError_t launch_attn_bwd_generic(const AttnDims& d, const void* q, const void* k,
                                   const void* v, const void* o, const float* lse,
                                   const void* dout, void* dq, void* dk, void* dv,
                                   float* delta_ws, hipStream_t stream) {
  GenParams p = make_params(d);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.out0 = dq;
  p.out1 = dk;
  p.out2 = dv;
  p.delta = delta_ws;
  if (d.dtype == 1) return d.D == 32 ? run_bwd<float, 32>(p, stream) : run_bwd<float, 64>(p, stream);
  return d.D == 32 ? run_bwd<bf16, 32>(p, stream) : run_bwd<bf16, 64>(p, stream);
}

}  // namespace bca
