// Short attention problems (at most 32 key positions, at most 64 folded
// query rows), bf16, head_dim 64: one wave per problem.
//
// Same definition as the other attention kernels (Open Dreamer articles,
// pro.edgex.exchange fr-FR edition, sections "Architecture" and
// "Configuration d'entraînement"): space attention inside one block with
// world tokens unable to read agent tokens, causal sliding-window time
// attention per token slot, GQA head h -> KV head h / (Hq / Hkv).  The shape
// that needs this path is the tokenizer's time layer (16 frames per clip,
// section "Configuration d'entraînement"): a problem there has 16 query rows
// and 16 keys, which the 256-row workgroups of the MFMA kernels would leave
// mostly idle.  The work per problem is tiny and the op is bound by HBM, so
// the arithmetic is fp32 on the vector units.
//
// A problem is (unit, KV head) with L key positions and R = L * G rows (row
// r = position * G + head in group), as in the MFMA kernels.  Lane l of the
// problem's wave holds row l / PARTS and the PARTS-th part of its 64 columns
// (PARTS = 64 / RP, RP = rows rounded up to 16, 32 or 64); a score is the sum
// of PARTS partial dot products over xor-shuffles.  K and V (and in the
// backward Q, dO, P and dS) are staged in the wave's own LDS slice.
//
//  short_fwd_kernel: every score (bf16 dot products on v_dot2), the masked
//      softmax in the log2 domain, O = P V (P as bf16, V transposed in LDS)
//      and LSE (natural log) per row.
//  short_bwd_kernel: phase A, lane = (row, part): P from the stored LSE,
//      Delta = rowsum(dO * O), dP = dO V^T, dS = P (dP - Delta), dQ = scale
//      dS K; phase B, lane = (key, part): dV = P^T dO, dK = scale dS^T Q,
//      summed over all rows of the problem (all G heads), so no atomics.
#include "bca_device.h"
#include "bca_kernels.h"

namespace bca {

namespace {

constexpr int SD = 64;      // head_dim of this path
constexpr int SWAVES = 4;   // problems (waves) per workgroup of the forward

// Problems per workgroup of the backward: its LDS slice per wave grows with
// rows x keys, and a workgroup may use at most 160 KB.
constexpr int bwd_waves(int RP, int LP) { return RP * LP >= 2048 ? 2 : 4; }

struct ShortParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const float* lse;
  const bf16* dout;
  bf16* out0;  // o (fwd) or dq (bwd)
  bf16* out1;  // dk
  bf16* out2;  // dv
  float* lse_out;
  int T, N, Hq, Hkv, G, L, R, problems;
  int window, agent_begin, agent_count;
  float scale;
  int poison;  // debug: NaN-fill LDS before staging
};

// Sum over the PARTS lanes of a row (adjacent lanes).
template <int PARTS>
__device__ __forceinline__ float part_sum(float x) {
  if constexpr (PARTS >= 2) x += __shfl_xor(x, 1, 64);
  if constexpr (PARTS >= 4) x += __shfl_xor(x, 2, 64);
  return x;
}

// Loads the L key rows of K and V of one problem into the wave's LDS slice
// ([LP][64] each); rows L .. LP-1 are zero.
template <int LP>
__device__ __forceinline__ void stage_kv(const bf16* kb, const bf16* vb, int64_t kstride, int L,
                                         int lane, bf16* sk, bf16* sv) {
#pragma unroll
  for (int it = 0; it < LP / 8; ++it) {
    const int j = it * 8 + (lane >> 3), c = (lane & 7) * 8;
    bf16x8 a = zero8(), b = zero8();
    if (j < L) {
      a = ld_global16(kb + (int64_t)j * kstride + c);
      b = ld_global16(vb + (int64_t)j * kstride + c);
    }
    st_lds16(sk + j * SD + c, a);
    st_lds16(sv + j * SD + c, b);
  }
}

template <int N>
__device__ __forceinline__ void load_f32(const bf16* p, float* f) {
#pragma unroll
  for (int c = 0; c < N; c += 8) {
    const bf16x8 x = ld_global16(p + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[c + e] = (float)x[e];
  }
}

template <int N>
__device__ __forceinline__ void store_bf16(bf16* p, const float* f) {
#pragma unroll
  for (int c = 0; c < N; c += 8) {
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (bf16)f[c + e];
    st_global16(p + c, x);
  }
}

// Partial dot product of `f` (this lane's DP columns) with LDS row `row`.
template <int DP>
__device__ __forceinline__ float dot_lds(const float* f, const bf16* row) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < DP; c += 8) {
    const bf16x8 x = ld_lds16(row + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = __builtin_fmaf(f[c + e], (float)x[e], s);
  }
  return s;
}

// The sum of the products of two bf16 vectors' 8 element pairs, added to s
// (v_dot2_f32_bf16: each bf16 product is exact in fp32).
__device__ __forceinline__ float dot8(const bf16x8& a, const bf16x8& b, float s) {
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), s, false);
  return s;
}

// Two passes over the problem's (at most 32) keys: every score first (the
// lane's partial dot products on v_dot2, summed over the row's lanes), then
// the row maximum, the exps and their sum, then O = P V with P rounded to
// bf16 (the matmul operand precision of the method, as on the MFMA path)
// and V read transposed from LDS, so that each output column is a bf16 dot
// product along the keys.
template <int OP, int RP, int LP>
__global__ __launch_bounds__(SWAVES * 64) void short_fwd_kernel(ShortParams p) {
  constexpr int PARTS = 64 / RP, DP = SD / PARTS;
  __shared__ __attribute__((aligned(16))) bf16 sK[SWAVES][LP * SD];
  __shared__ __attribute__((aligned(16))) bf16 sVt[SWAVES][SD * LP];  // [column][key]
  if (p.poison) {
    poison_lds(sK, sizeof(sK), threadIdx.x, SWAVES * 64);
    poison_lds(sVt, sizeof(sVt), threadIdx.x, SWAVES * 64);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int prob = blockIdx.x * SWAVES + wave;
  const bool live = prob < p.problems;  // uniform per wave
  const int u = live ? prob / p.Hkv : 0, g = live ? prob - u * p.Hkv : 0;
  const UnitGeom gq = unit_geom(OP, u, p.T, p.N, p.Hq, SD);
  const UnitGeom gk = unit_geom(OP, u, p.T, p.N, p.Hkv, SD);
  const UnitGeom gl = unit_geom(OP, u, p.T, p.N, p.Hq, 1);
  if (live) {
    // K row-major, V transposed (rows past L are zero)
    const bf16* kb = p.k + gk.base + (int64_t)g * SD;
    const bf16* vb = p.v + gk.base + (int64_t)g * SD;
#pragma unroll
    for (int it = 0; it < LP / 8; ++it) {
      const int j = it * 8 + (lane >> 3), c = (lane & 7) * 8;
      bf16x8 a = zero8(), b = zero8();
      if (j < p.L) {
        a = ld_global16(kb + (int64_t)j * gk.pos_stride + c);
        b = ld_global16(vb + (int64_t)j * gk.pos_stride + c);
      }
      st_lds16(sK[wave] + j * SD + c, a);
#pragma unroll
      for (int t = 0; t < 8; ++t) sVt[wave][(c + t) * LP + j] = b[t];
    }
  }
  __syncthreads();
  if (!live) return;

  const int r = lane / PARTS, part = lane % PARTS;
  const bool row_ok = r < p.R;
  const int pos = row_ok ? r / p.G : 0, hd = g * p.G + (row_ok ? r % p.G : 0);
  const int64_t qoff = gq.base + (int64_t)pos * gq.pos_stride + (int64_t)hd * SD + part * DP;
  bf16x8 qv[DP / 8];
#pragma unroll
  for (int c = 0; c < DP / 8; ++c) qv[c] = ld_global16(p.q + qoff + c * 8);
  const MaskDesc md{OP, p.L, p.window, p.agent_begin, p.agent_count};
  const float c2 = p.scale * kLog2e;
  float sc[LP];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < LP; ++j) {
    const bf16* kr = sK[wave] + j * SD + part * DP;
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int c = 0; c < DP / 8; c += 2) {
      d0 = dot8(qv[c], ld_lds16(kr + c * 8), d0);
      if (c + 1 < DP / 8) d1 = dot8(qv[c + 1], ld_lds16(kr + (c + 1) * 8), d1);
    }
    const float d = part_sum<PARTS>(d0 + d1);
    sc[j] = (j < p.L && visible_op<OP>(md, pos, j)) ? d * c2 : -INFINITY;
    m = fmaxf(m, sc[j]);
  }
  // every row sees at least its own position, so m is finite
  float l = 0.f;
#pragma unroll
  for (int j = 0; j < LP; ++j) {
    sc[j] = fast_exp2(sc[j] - m);
    l += sc[j];
  }
  bf16x8 pb[LP / 8];
#pragma unroll
  for (int i = 0; i < LP / 8; ++i)
    pb[i] = pack8(f32x4{sc[8 * i], sc[8 * i + 1], sc[8 * i + 2], sc[8 * i + 3]},
                  f32x4{sc[8 * i + 4], sc[8 * i + 5], sc[8 * i + 6], sc[8 * i + 7]});
  const float inv = 1.f / l;
  float acc[DP];
#pragma unroll
  for (int c = 0; c < DP; ++c) {
    const bf16* vr = sVt[wave] + (part * DP + c) * LP;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int i = 0; i < LP / 8; i += 2) {
      a0 = dot8(pb[i], ld_lds16(vr + i * 8), a0);
      if (i + 1 < LP / 8) a1 = dot8(pb[i + 1], ld_lds16(vr + (i + 1) * 8), a1);
    }
    acc[c] = (a0 + a1) * inv;
  }
  if (!row_ok) return;
  store_bf16<DP>(p.out0 + qoff, acc);
  if (part == 0) p.lse_out[gl.base + (int64_t)pos * gl.pos_stride + hd] = (m + log2f(l)) * kLn2;
}

template <int OP, int RP, int LP>
__global__ __launch_bounds__(bwd_waves(RP, LP) * 64) void short_bwd_kernel(ShortParams p) {
  constexpr int SWAVES = bwd_waves(RP, LP);
  constexpr int PARTS = 64 / RP, DP = SD / PARTS;      // phase A: lane = (row, part)
  constexpr int KPARTS = 64 / LP, KDP = SD / KPARTS;   // phase B: lane = (key, part)
  __shared__ __attribute__((aligned(16))) bf16 sK[SWAVES][LP * SD];
  __shared__ __attribute__((aligned(16))) bf16 sV[SWAVES][LP * SD];
  __shared__ __attribute__((aligned(16))) bf16 sQ[SWAVES][RP * SD];
  __shared__ __attribute__((aligned(16))) bf16 sO[SWAVES][RP * SD];  // dO rows
  __shared__ float sP[SWAVES][LP * RP];                                // [key][row]
  __shared__ float sS[SWAVES][LP * RP];                                // dS, [key][row]
  if (p.poison) {
    constexpr int NT = SWAVES * 64;
    poison_lds(sK, sizeof(sK), threadIdx.x, NT);
    poison_lds(sV, sizeof(sV), threadIdx.x, NT);
    poison_lds(sQ, sizeof(sQ), threadIdx.x, NT);
    poison_lds(sO, sizeof(sO), threadIdx.x, NT);
    poison_lds(sP, sizeof(sP), threadIdx.x, NT);
    poison_lds(sS, sizeof(sS), threadIdx.x, NT);
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int prob = blockIdx.x * SWAVES + wave;
  const bool live = prob < p.problems;
  const int u = live ? prob / p.Hkv : 0, g = live ? prob - u * p.Hkv : 0;
  const UnitGeom gq = unit_geom(OP, u, p.T, p.N, p.Hq, SD);
  const UnitGeom gk = unit_geom(OP, u, p.T, p.N, p.Hkv, SD);
  const UnitGeom gl = unit_geom(OP, u, p.T, p.N, p.Hq, 1);
  if (live)
    stage_kv<LP>(p.k + gk.base + (int64_t)g * SD, p.v + gk.base + (int64_t)g * SD, gk.pos_stride,
                 p.L, lane, sK[wave], sV[wave]);
  __syncthreads();

  // ---- phase A: one row per PARTS lanes
  if (live) {
    const int r = lane / PARTS, part = lane % PARTS;
    const bool row_ok = r < p.R;
    const int pos = row_ok ? r / p.G : 0, hd = g * p.G + (row_ok ? r % p.G : 0);
    const int64_t off = gq.base + (int64_t)pos * gq.pos_stride + (int64_t)hd * SD + part * DP;
    float qf[DP], df[DP];
    float delta;
    {
      float of[DP];
      load_f32<DP>(p.q + off, qf);
      load_f32<DP>(p.dout + off, df);
      load_f32<DP>(p.o + off, of);
      float t = 0.f;
#pragma unroll
      for (int c = 0; c < DP; ++c) t = __builtin_fmaf(df[c], of[c], t);
      delta = part_sum<PARTS>(t);
    }
    const float lse2 = row_ok ? p.lse[gl.base + (int64_t)pos * gl.pos_stride + hd] * kLog2e : 0.f;
    const MaskDesc md{OP, p.L, p.window, p.agent_begin, p.agent_count};
    const float c2 = p.scale * kLog2e;
    float dq[DP];
#pragma unroll
    for (int c = 0; c < DP; ++c) dq[c] = 0.f;
#pragma unroll 2
    for (int j = 0; j < p.L; ++j) {
      const float sc = part_sum<PARTS>(dot_lds<DP>(qf, sK[wave] + j * SD + part * DP));
      const float dp = part_sum<PARTS>(dot_lds<DP>(df, sV[wave] + j * SD + part * DP));
      const bool vis = row_ok && visible_op<OP>(md, pos, j);
      const float pr = vis ? fast_exp2(sc * c2 - lse2) : 0.f;
      const float ds = pr * (dp - delta);
      const bf16* kr = sK[wave] + j * SD + part * DP;
#pragma unroll
      for (int c = 0; c < DP; c += 8) {
        const bf16x8 x = ld_lds16(kr + c);
#pragma unroll
        for (int e = 0; e < 8; ++e) dq[c + e] = __builtin_fmaf(ds, (float)x[e], dq[c + e]);
      }
      // every lane of the row holds pr and ds; lane `part` stores keys j
      // with j % PARTS == part
      if (j % PARTS == part) {
        sP[wave][j * RP + r] = pr;
        sS[wave][j * RP + r] = ds;
      }
    }
    // rows past R are zero in sQ / sO (their P and dS are zero too)
    {
      float z[DP];
#pragma unroll
      for (int c = 0; c < DP; ++c) z[c] = row_ok ? qf[c] : 0.f;
#pragma unroll
      for (int c = 0; c < DP; c += 8) {
        bf16x8 x, y;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[e] = (bf16)z[c + e];
          y[e] = (bf16)(row_ok ? df[c + e] : 0.f);
        }
        st_lds16(sQ[wave] + r * SD + part * DP + c, x);
        st_lds16(sO[wave] + r * SD + part * DP + c, y);
      }
    }
    if (row_ok) {
#pragma unroll
      for (int c = 0; c < DP; ++c) dq[c] *= p.scale;
      store_bf16<DP>(p.out0 + off, dq);
    }
  }
  __syncthreads();

  // ---- phase B: one key per KPARTS lanes, sums over every row of the problem
  if (!live) return;
  const int j = lane / KPARTS, part = lane % KPARTS;
  if (j >= p.L) return;
  float dk[KDP], dv[KDP];
#pragma unroll
  for (int c = 0; c < KDP; ++c) dk[c] = dv[c] = 0.f;
  for (int r = 0; r < p.R; ++r) {
    const float pr = sP[wave][j * RP + r], ds = sS[wave][j * RP + r];
    const bf16* qr = sQ[wave] + r * SD + part * KDP;
    const bf16* orow = sO[wave] + r * SD + part * KDP;
#pragma unroll
    for (int c = 0; c < KDP; c += 8) {
      const bf16x8 x = ld_lds16(qr + c), y = ld_lds16(orow + c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dk[c + e] = __builtin_fmaf(ds, (float)x[e], dk[c + e]);
        dv[c + e] = __builtin_fmaf(pr, (float)y[e], dv[c + e]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < KDP; ++c) dk[c] *= p.scale;
  const int64_t koff = gk.base + (int64_t)j * gk.pos_stride + (int64_t)g * SD + part * KDP;
  store_bf16<KDP>(p.out1 + koff, dk);
  store_bf16<KDP>(p.out2 + koff, dv);
}

ShortParams make_short(const AttnDims& d) {
  ShortParams p{};
  p.T = d.T;
  p.N = d.N;
  p.Hq = d.Hq;
  p.Hkv = d.Hkv;
  p.G = d.Hq / d.Hkv;
  p.L = d.op == OP_SPACE ? d.N : d.T;
  p.R = p.L * p.G;
  p.problems = (d.op == OP_SPACE ? d.B * d.T : d.B * d.N) * d.Hkv;
  p.window = d.window;
  p.agent_begin = d.agent_begin;
  p.agent_count = d.agent_count;
  p.scale = d.scale;
  p.poison = d.poison;
  return p;
}

template <template <int, int, int> class K, int OP, int RP, int LP>
hipError_t launch_one(const ShortParams& p, hipStream_t stream) {
  constexpr int W = K<OP, RP, LP>::waves;
  const int64_t blocks = ((int64_t)p.problems + W - 1) / W;
  if (blocks <= 0 || blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((K<OP, RP, LP>::fn), dim3((unsigned)blocks), dim3(W * 64), 0, stream, p);
  return hipGetLastError();
}

// Instance by (rows, keys): R <= 16 and L <= 16; R <= 32 and L <= 32;
// otherwise R <= 64 with 16 or 32 keys.
template <template <int, int, int> class K, int OP>
hipError_t launch_short_op(const ShortParams& p, hipStream_t stream) {
  if (p.R <= 16) return launch_one<K, OP, 16, 16>(p, stream);
  if (p.R <= 32) return launch_one<K, OP, 32, 32>(p, stream);
  if (p.L <= 16) return launch_one<K, OP, 64, 16>(p, stream);
  return launch_one<K, OP, 64, 32>(p, stream);
}

template <int OP, int RP, int LP>
struct FwdK {
  static constexpr auto fn = short_fwd_kernel<OP, RP, LP>;
  static constexpr int waves = SWAVES;
};
template <int OP, int RP, int LP>
struct BwdK {
  static constexpr auto fn = short_bwd_kernel<OP, RP, LP>;
  static constexpr int waves = bwd_waves(RP, LP);
};

}  // namespace

hipError_t launch_attn_fwd_short(const AttnDims& d, const void* q, const void* k, const void* v,
                                 void* o, float* lse, hipStream_t stream) {
  ShortParams p = make_short(d);
  p.q = static_cast<const bf16*>(q);
  p.k = static_cast<const bf16*>(k);
  p.v = static_cast<const bf16*>(v);
  p.out0 = static_cast<bf16*>(o);
  p.lse_out = lse;
  return d.op == OP_SPACE ? launch_short_op<FwdK, OP_SPACE>(p, stream)
                          : launch_short_op<FwdK, OP_TIME>(p, stream);
}

hipError_t launch_attn_bwd_short(const AttnDims& d, const void* q, const void* k, const void* v,
                                 const void* o, const float* lse, const void* dout, void* dq,
                                 void* dk, void* dv, hipStream_t stream) {
  ShortParams p = make_short(d);
  p.q = static_cast<const bf16*>(q);
  p.k = static_cast<const bf16*>(k);
  p.v = static_cast<const bf16*>(v);
  p.o = static_cast<const bf16*>(o);
  p.lse = lse;
  p.dout = static_cast<const bf16*>(dout);
  p.out0 = static_cast<bf16*>(dq);
  p.out1 = static_cast<bf16*>(dk);
  p.out2 = static_cast<bf16*>(dv);
  return d.op == OP_SPACE ? launch_short_op<BwdK, OP_SPACE>(p, stream)
                          : launch_short_op<BwdK, OP_TIME>(p, stream);
}

}  // namespace bca
