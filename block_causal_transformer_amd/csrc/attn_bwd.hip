// Backward of space and time attention, bf16 in/out, head_dim 64, for
// problems of at most 320 positions (the dynamics model's 290-token blocks
// and 256-frame slots), on gfx950.
//
// Open Dreamer articles (pro.edgex.exchange, fr-FR edition), sections
// "Architecture" and "Configuration d'entraînement" (masks, GQA), and section
// "Performance de calcul et stratégie mémoire" (activation checkpointing): the
// forward keeps only O and the fp32 log-sum-exp, and the backward recomputes
// the probabilities from them.
//
// Gradients of L = sum(O * dO):
//   Delta_i = <dO_i, O_i>,  P = exp(s Q K^T - LSE),  dP = dO V^T,
//   dS = P o (dP - Delta),  dV = P^T dO,  dK = s dS^T Q,  dQ = s dS K,
// with dK, dV of a KV head summed over the G query heads of its group.
//
// Decomposition.  One workgroup (4 waves) owns a whole (unit, KV head)
// problem, so every sum stays inside it and no atomics are needed; the result
// is bitwise deterministic.  Keys are cut into 16-key tiles dealt round-robin
// to the waves; each wave keeps its tiles' K and V (as MFMA operands) and its
// dK^T, dV^T accumulators in registers for the whole kernel.  The problem's
// rows (position x head-in-group, as in the forward) are swept in 32-row
// chunks:
//   1. all threads stage Q, dO (row-major and transposed) and LSE of the
//      chunk in LDS and compute Delta from O and dO on the fly (no separate
//      pre-pass kernel, O is read exactly once);
//   2. each wave, per own key tile: S and dP on MFMA, P and dS on VALU,
//      dV^T += dO^T P and dK^T += Q^T dS on MFMA, and dS written to LDS;
//   3. dQ^T = K^T dS^T for the chunk from LDS (K^T staged once), split over
//      the waves by output tile, written straight to HBM.
// Key tiles a chunk cannot see (causal and window ranges) are skipped.
#include "bca_device.h"
#include "bca_kernels.h"

namespace bca {

namespace {

constexpr int KMAX = kMfmaBwdMaxLen;  // 320
constexpr int QC = 32;                // rows per chunk
constexpr int KTW = KMAX / 16 / 4;    // 16-key tiles per wave (5)

struct BwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const float* lse;
  const bf16* dout;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  int op, T, N, Hq, Hkv, G, L, units, rows;
  int window, agent_begin, agent_count;
  float scale, scale_log2;
};

__device__ __forceinline__ int kt_off(int d, int key) {  // sKT: [64][KMAX]
  return d * KMAX + ((((key >> 3) ^ (d & 7))) << 3) + (key & 7);
}
__device__ __forceinline__ int ds_off(int q, int key) {  // sdS: [QC][KMAX]
  return q * KMAX + ((((key >> 3) ^ (q & 7))) << 3) + (key & 7);
}
__device__ __forceinline__ int row_off(int row, int chunk) {  // sQ, sdO: [QC][64]
  return row * 64 + ((chunk ^ (row & 7)) << 3);
}
// Transposed chunk rows: query q of the chunk sits at position
// 8*((q>>2)&3) + 4*(q>>4) + (q&3), so the 8 queries a lane feeds to one
// MFMA (q = 16h + 4g + j) are contiguous.
__device__ __forceinline__ int tq_perm(int q) {
  return (((q >> 2) & 3) << 3) | ((q >> 4) << 2) | (q & 3);
}
__device__ __forceinline__ int tr_off(int d, int pos) {  // sQT, sdOT: [64][QC]
  return d * QC + ((((pos >> 3) ^ (d & 3))) << 3) + (pos & 7);
}

__global__ __launch_bounds__(256, 1) void attn_bwd_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) bf16 sKT[64 * KMAX];
  __shared__ __attribute__((aligned(16))) bf16 sdS[QC * KMAX];
  __shared__ __attribute__((aligned(16))) bf16 sQ[QC * 64];
  __shared__ __attribute__((aligned(16))) bf16 sdO[QC * 64];
  __shared__ __attribute__((aligned(16))) bf16 sQT[64 * QC];
  __shared__ __attribute__((aligned(16))) bf16 sdOT[64 * QC];
  __shared__ __attribute__((aligned(16))) float sLse[QC];
  __shared__ __attribute__((aligned(16))) float sDelta[QC];

  const int ug = blockIdx.x;
  const int u = ug / p.Hkv, g = ug - (ug / p.Hkv) * p.Hkv;
  const UnitGeom gq = unit_geom(p.op, u, p.T, p.N, p.Hq, 64);
  const UnitGeom gk = unit_geom(p.op, u, p.T, p.N, p.Hkv, 64);
  const UnitGeom gl = unit_geom(p.op, u, p.T, p.N, p.Hq, 1);
  const MaskDesc md{p.op, p.L, p.window, p.agent_begin, p.agent_count};
  const int G = p.G;
  const int64_t qhead = (int64_t)g * G * 64;
  const bf16* kbase = p.k + gk.base + g * 64;
  const bf16* vbase = p.v + gk.base + g * 64;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int nkt = (p.L + 15) >> 4;
  const int lp32 = (p.L + 31) & ~31;

  // K^T of the problem in LDS (zero beyond L), for the dQ product.
  for (int idx = tid; idx < lp32 * 8; idx += 256) {
    const int r = idx >> 3, c = idx & 7;
    const bf16x8 kv = r < p.L ? ld_global16(kbase + (int64_t)r * gk.pos_stride + c * 8) : zero8();
#pragma unroll
    for (int e = 0; e < 8; ++e) sKT[kt_off(c * 8 + e, r)] = kv[e];
  }
  // dS columns of the padding tile (never written by the waves) stay zero.
  for (int idx = tid; idx < QC * (lp32 - nkt * 16); idx += 256) {
    const int qrow = idx / (lp32 - nkt * 16), col = nkt * 16 + idx % (lp32 - nkt * 16);
    sdS[ds_off(qrow, col)] = (bf16)0.f;
  }

  // Own key tiles: kt = wave + 4*m.  K and V as B operands (column = key).
  bf16x8 KB[KTW][2], VB[KTW][2];
  f32x4 dKT[KTW][4], dVT[KTW][4];
#pragma unroll
  for (int m = 0; m < KTW; ++m) {
    const int key = (wave + 4 * m) * 16 + li;
    const bool ok = key < p.L;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      KB[m][s] = ok ? ld_global16(kbase + (int64_t)key * gk.pos_stride + s * 32 + lg * 8) : zero8();
      VB[m][s] = ok ? ld_global16(vbase + (int64_t)key * gk.pos_stride + s * 32 + lg * 8) : zero8();
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      dKT[m][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dVT[m][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  const int nchunks = (p.rows + QC - 1) / QC;
  for (int c = 0; c < nchunks; ++c) {
    const int r0 = c * QC;
    // ---- 1. stage the chunk (one 16-byte piece of Q, dO, O per thread)
    {
      const int row = tid >> 3, ch = tid & 7;
      const int r = r0 + row;
      const bool valid = r < p.rows;
      const int pos = valid ? r / G : 0;
      const int hh = valid ? r - pos * G : 0;
      const int64_t off = gq.base + (int64_t)pos * gq.pos_stride + qhead + hh * 64 + ch * 8;
      const bf16x8 qv = valid ? ld_global16(p.q + off) : zero8();
      const bf16x8 dov = valid ? ld_global16(p.dout + off) : zero8();
      const bf16x8 ov = valid ? ld_global16(p.o + off) : zero8();
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) part += (float)dov[e] * (float)ov[e];
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      part += __shfl_xor(part, 4);
      st_lds16(sQ + row_off(row, ch), qv);
      st_lds16(sdO + row_off(row, ch), dov);
      const int tp = tq_perm(row);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sQT[tr_off(ch * 8 + e, tp)] = qv[e];
        sdOT[tr_off(ch * 8 + e, tp)] = dov[e];
      }
      if (ch == 0) {
        sDelta[row] = part;
        sLse[row] = valid ? p.lse[gl.base + (int64_t)pos * gl.pos_stride + g * G + hh] * kLog2e
                          : INFINITY;
      }
    }
    __syncthreads();

    // ---- 2. per-wave key tiles
    const int qlo = r0 / G;
    const int qhi = (min(r0 + QC, p.rows) - 1) / G;
    int klo, khi;
    key_range(md, qlo, qhi, klo, khi);
    const int step_lo = klo >> 5, step_hi = (khi + 31) >> 5;  // dQ key steps
    {
      bf16x8 Qa[2][2], dOa[2][2], QTa[4], dOTa[4];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          Qa[qt][s] = ld_lds16(sQ + row_off(qt * 16 + li, s * 4 + lg));
          dOa[qt][s] = ld_lds16(sdO + row_off(qt * 16 + li, s * 4 + lg));
        }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        QTa[dt] = ld_lds16(sQT + tr_off(dt * 16 + li, lg * 8));
        dOTa[dt] = ld_lds16(sdOT + tr_off(dt * 16 + li, lg * 8));
      }
      f32x4 lse4[2], dl4[2];
      int qpr[2][4];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        lse4[qt] = *reinterpret_cast<const f32x4*>(sLse + qt * 16 + lg * 4);
        dl4[qt] = *reinterpret_cast<const f32x4*>(sDelta + qt * 16 + lg * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) qpr[qt][j] = (r0 + qt * 16 + lg * 4 + j) / G;
      }

#pragma unroll
      for (int m = 0; m < KTW; ++m) {
        const int kt = wave + 4 * m;
        if (kt >= nkt) break;
        const int kabs = kt * 16;
        if (kabs + 16 <= klo || kabs >= khi || tile_none_visible(md, qlo, qhi, kabs, kabs + 16)) {
          if (kabs < step_hi * 32 && kabs + 16 > step_lo * 32) {
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
              for (int j = 0; j < 4; ++j) sdS[ds_off(qt * 16 + lg * 4 + j, kabs + li)] = (bf16)0.f;
          }
          continue;
        }
        f32x4 S[2], dP[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
          z = mfma16(Qa[qt][0], KB[m][0], z);
          S[qt] = mfma16(Qa[qt][1], KB[m][1], z);
          f32x4 y = {0.f, 0.f, 0.f, 0.f};
          y = mfma16(dOa[qt][0], VB[m][0], y);
          dP[qt] = mfma16(dOa[qt][1], VB[m][1], y);
        }
        const bool full = tile_all_visible(md, qlo, qhi, kabs, kabs + 16);
        f32x4 P[2], dS[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool vis = full || visible(md, qpr[qt][j], kabs + li);
            const float e = fast_exp2(__builtin_fmaf(S[qt][j], p.scale_log2, -lse4[qt][j]));
            const float pv = vis ? e : 0.f;
            P[qt][j] = pv;
            dS[qt][j] = pv * (dP[qt][j] - dl4[qt][j]);
          }
        const bf16x8 Pb = pack8(P[0], P[1]);
        const bf16x8 dSb = pack8(dS[0], dS[1]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          dVT[m][dt] = mfma16(dOTa[dt], Pb, dVT[m][dt]);
          dKT[m][dt] = mfma16(QTa[dt], dSb, dKT[m][dt]);
        }
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int j = 0; j < 4; ++j) sdS[ds_off(qt * 16 + lg * 4 + j, kabs + li)] = dSb[qt * 4 + j];
      }
    }
    __syncthreads();

    // ---- 3. dQ^T = K^T dS^T: wave w computes query tile (w & 1) for the two
    // 16-wide head-dim tiles 2*(w >> 1) and 2*(w >> 1) + 1.
    {
      const int qt = wave & 1, dt0 = (wave >> 1) * 2;
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
      for (int st = step_lo; st < step_hi; ++st) {
        const bf16x8 b = ld_lds16(sdS + ds_off(qt * 16 + li, st * 32 + lg * 8));
        const bf16x8 k0 = ld_lds16(sKT + kt_off(dt0 * 16 + li, st * 32 + lg * 8));
        const bf16x8 k1 = ld_lds16(sKT + kt_off(dt0 * 16 + 16 + li, st * 32 + lg * 8));
        a0 = mfma16(k0, b, a0);
        a1 = mfma16(k1, b, a1);
      }
      const int r = r0 + qt * 16 + li;
      if (r < p.rows) {
        const int pos = r / G, hh = r - (r / G) * G;
        bf16* dst = p.dq + gq.base + (int64_t)pos * gq.pos_stride + qhead + hh * 64 + lg * 4;
        *reinterpret_cast<u32x2*>(dst + dt0 * 16) = __builtin_bit_cast(u32x2, pack4(a0 * p.scale));
        *reinterpret_cast<u32x2*>(dst + dt0 * 16 + 16) = __builtin_bit_cast(u32x2, pack4(a1 * p.scale));
      }
    }
    // The next chunk's staging writes sQ/sdO/sQT/sdOT/sLse/sDelta only,
    // which no wave reads after the barrier above; its barrier then orders
    // these dS reads before the next chunk's dS writes.
  }

  // ---- dK, dV of the own tiles: lane holds column key, rows d = dt*16 + lg*4 + j
#pragma unroll
  for (int m = 0; m < KTW; ++m) {
    const int key = (wave + 4 * m) * 16 + li;
    if (key >= p.L) continue;
    bf16* dkd = p.dk + gk.base + (int64_t)key * gk.pos_stride + g * 64 + lg * 4;
    bf16* dvd = p.dv + gk.base + (int64_t)key * gk.pos_stride + g * 64 + lg * 4;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      *reinterpret_cast<u32x2*>(dkd + dt * 16) = __builtin_bit_cast(u32x2, pack4(dKT[m][dt] * p.scale));
      *reinterpret_cast<u32x2*>(dvd + dt * 16) = __builtin_bit_cast(u32x2, pack4(dVT[m][dt]));
    }
  }
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const AttnDims& d, const void* q, const void* k, const void* v,
                                const void* o, const float* lse, const void* dout, void* dq,
                                void* dk, void* dv, hipStream_t stream) {
  BwdParams p;
  p.q = static_cast<const bf16*>(q);
  p.k = static_cast<const bf16*>(k);
  p.v = static_cast<const bf16*>(v);
  p.o = static_cast<const bf16*>(o);
  p.lse = lse;
  p.dout = static_cast<const bf16*>(dout);
  p.dq = static_cast<bf16*>(dq);
  p.dk = static_cast<bf16*>(dk);
  p.dv = static_cast<bf16*>(dv);
  p.op = d.op;
  p.T = d.T;
  p.N = d.N;
  p.Hq = d.Hq;
  p.Hkv = d.Hkv;
  p.G = d.Hq / d.Hkv;
  p.L = d.op == OP_SPACE ? d.N : d.T;
  p.units = d.op == OP_SPACE ? d.B * d.T : d.B * d.N;
  p.rows = p.L * p.G;
  p.window = d.window;
  p.agent_begin = d.agent_begin;
  p.agent_count = d.agent_count;
  p.scale = d.scale;
  p.scale_log2 = d.scale * kLog2e;
  if (p.L > KMAX) return hipErrorInvalidValue;
  const long grid = (long)p.units * p.Hkv;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_bwd_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace bca
