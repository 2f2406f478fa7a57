// Device-side helpers shared by the gfx950 attention kernels.
//
// MFMA used throughout: v_mfma_f32_16x16x32_bf16 (16x16 output tile, 32-deep
// contraction, 8 bf16 per lane per operand, fp32 accumulate).  For lane l let
// i = l % 16 and g = l / 16.  Operand A (16 x 32) holds row i, operand B
// (32 x 16) holds column i; the 8 values of a lane cover 8 of the 32
// contraction indices, and any bijection (g, e) -> k works as long as A and B
// use the same one.  The kernels choose that bijection per product so that
// every operand is one 16-byte LDS or global read.  The output tile holds
// C[g*4 + j][i], j = 0..3, in the lane's 4 fp32 registers.
//
// The dQ step of the three-slot backward uses v_mfma_f32_32x32x16_bf16
// (32x32 output, 16-deep): lane l holds row l % 32 of A and column l % 32
// of B for contraction indices 8 (l / 32) .. +7, and output rows
// 8 (i / 4) + 4 (l / 32) + i % 4 (i < 16) of column l % 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bca {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// OP_DECODE: time attention of a few new frames against a ring-buffer cache
// of earlier frames' K/V (rollout); its masks are the time op's.
enum OpKind { OP_SPACE = 0, OP_TIME = 1, OP_DECODE = 2 };

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum over the four lanes that share i = lane % 16 (g = 0..3), using
// the gfx950 row-swap permutes.  With both operands equal to x,
// permlane16_swap returns {x of rows (0,0,2,2), x of rows (1,1,3,3)} (16-lane
// rows), so the pair always holds a lane's own value and its partner's in
// the adjacent row; permlane32_swap does the same for the two 32-lane halves.
__device__ __forceinline__ float group4_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float group4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Pack 8 fp32 values into a bf16x8 operand (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(const f32x4& a, const f32x4& b) {
  bf16x8 r;
  r[0] = (bf16)a[0]; r[1] = (bf16)a[1]; r[2] = (bf16)a[2]; r[3] = (bf16)a[3];
  r[4] = (bf16)b[0]; r[5] = (bf16)b[1]; r[6] = (bf16)b[2]; r[7] = (bf16)b[3];
  return r;
}

__device__ __forceinline__ bf16x4 pack4(const f32x4& a) {
  bf16x4 r;
  r[0] = (bf16)a[0]; r[1] = (bf16)a[1]; r[2] = (bf16)a[2]; r[3] = (bf16)a[3];
  return r;
}

__device__ __forceinline__ bf16x8 zero8() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, z);
}

__device__ __forceinline__ bf16x8 ld_global16(const bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 ld_lds16(const bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void st_global16(bf16* p, const bf16x8& v) {
  *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, v);
}

__device__ __forceinline__ void st_lds16(bf16* p, const bf16x8& v) {
  *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, v);
}

// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Within each group of
// 16 lanes, lane i receives as its element e the element (i & 3) of the
// 8-byte piece addressed by lane 4*e + (i >> 2) of the same group.  So if
// lane s addresses row R(s >> 2), columns c0 + 4*(s & 3) .. +3 of a
// row-major bf16 tile, lane i receives column c0 + i of rows R(0..3): four
// rows of one column, as an MFMA operand wants them.
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x4 ld_lds_tr4(const bf16* p) {
  typedef __attribute__((address_space(3))) i16x4* lds_i16x4_ptr;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// Debug aid: fill `bytes` (a multiple of 16) of LDS at `p` with all-ones
// words, a NaN in both bf16 and fp32, from the `nthreads` threads of the
// workgroup.  The caller places a barrier between this and the first staging.
__device__ __forceinline__ void poison_lds(void* p, int bytes, int tid, int nthreads) {
  const u32x4 nan4 = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
  u32x4* w = reinterpret_cast<u32x4*>(p);
  for (int i = tid; i < bytes / 16; i += nthreads) w[i] = nan4;
}

__device__ __forceinline__ bf16x8 join8(const bf16x4& a, const bf16x4& b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Element offsets of position 0 of a unit (a block for space attention, a
// token slot for time attention) for a tensor with H heads of width D, and
// the stride between positions.  Tensors are (B, T, N, H, D) row-major.
struct UnitGeom {
  int64_t base;
  int64_t pos_stride;
};

__device__ __forceinline__ UnitGeom unit_geom(int op, int u, int T, int N, int H, int D) {
  UnitGeom g;
  if (op == OP_SPACE) {
    g.base = (int64_t)u * N * H * D;
    g.pos_stride = (int64_t)H * D;
  } else {
    const int b = u / N, n = u - (u / N) * N;
    g.base = ((int64_t)b * T * N + n) * H * D;
    g.pos_stride = (int64_t)N * H * D;
  }
  return g;
}

// Visibility of key position kp to a query at position qp.  Space: world
// queries cannot see agent keys; padding keys (kp >= L) are never visible.
// Time: causal with an optional sliding window that counts the current frame.
struct MaskDesc {
  int op, L, window, agent_begin, agent_count;
};

__device__ __forceinline__ bool visible(const MaskDesc& m, int qp, int kp) {
  if (kp >= m.L) return false;
  if (m.op == OP_TIME) {
    if (kp > qp) return false;
    if (m.window > 0 && qp - kp >= m.window) return false;
    return true;
  }
  const bool ka = (unsigned)(kp - m.agent_begin) < (unsigned)m.agent_count;
  const bool qa = (unsigned)(qp - m.agent_begin) < (unsigned)m.agent_count;
  return !(ka && !qa);
}

// Branch-free form of visible() for a mask kind fixed at compile time.
template <int OP>
__device__ __forceinline__ bool visible_op(const MaskDesc& m, int qp, int kp) {
  if constexpr (OP == OP_TIME) {
    return (kp <= qp) & (kp < m.L) & ((m.window == 0) | (qp - kp < m.window));
  } else {
    const bool ka = (unsigned)(kp - m.agent_begin) < (unsigned)m.agent_count;
    const bool qa = (unsigned)(qp - m.agent_begin) < (unsigned)m.agent_count;
    return (kp < m.L) & !(ka & !qa);
  }
}

// Position (row / G) of a folded row index, exact for rows < 2^21 and
// G <= 256: (r + 0.5) / G keeps a margin of 0.5/G from the next integer,
// more than the two fp32 roundings can move it.
__device__ __forceinline__ int row_pos(int r, float inv_g) {
  return (int)(((float)r + 0.5f) * inv_g);
}

// Key-position range [lo, hi) that any query position in [qlo, qhi] can see.
__device__ __forceinline__ void key_range(const MaskDesc& m, int qlo, int qhi, int& lo, int& hi) {
  if (m.op == OP_TIME) {
    lo = (m.window > 0) ? max(0, qlo - m.window + 1) : 0;
    hi = min(m.L, qhi + 1);
  } else {
    lo = 0;
    hi = m.L;
  }
}

// True when every (query in [qlo, qhi], key in [klo, khi)) pair is visible,
// so a tile needs no per-element mask.
__device__ __forceinline__ bool tile_all_visible(const MaskDesc& m, int qlo, int qhi, int klo, int khi) {
  if (khi > m.L) return false;
  if (m.op == OP_TIME) {
    if (khi - 1 > qlo) return false;
    if (m.window > 0 && qhi - klo >= m.window) return false;
    return true;
  }
  if (m.agent_count == 0) return true;
  const int ab = m.agent_begin, ae = m.agent_begin + m.agent_count;
  if (khi <= ab || klo >= ae) return true;
  // the tile touches agent keys: fine only if every query is an agent
  return qlo >= ab && qhi < ae;
}

// True when no pair in the tile is visible.
__device__ __forceinline__ bool tile_none_visible(const MaskDesc& m, int qlo, int qhi, int klo, int khi) {
  if (klo >= m.L) return true;
  if (m.op == OP_TIME) {
    if (klo > qhi) return true;
    if (m.window > 0 && qlo - (khi - 1) >= m.window) return true;
    return false;
  }
  return false;
}

// XCD-aware block order: the hardware deals consecutive workgroup ids to the
// 8 XCDs in turn.  Map the dispatch id so that the `inner` workgroups that
// share one (unit, KV head) land on the same XCD (and its L2).
__device__ __forceinline__ void xcd_remap(int bid, int outer, int inner, int& o, int& in) {
  const int full = (outer / 8) * 8;
  const int per8 = 8 * inner;
  if (bid < full * inner) {
    const int grp = bid / per8, r = bid - grp * per8;
    in = r / 8;
    o = grp * 8 + (r - in * 8);
  } else {
    const int r = bid - full * inner;
    const int rem = outer - full;
    in = r / rem;
    o = full + (r - in * rem);
  }
}

}  // namespace bca
