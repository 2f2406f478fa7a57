// Backward of space and time attention, bf16 in/out, head_dim 64, on gfx950.
// Problems of up to 320 positions (the dynamics model's 290-token blocks and
// 256-frame slots) keep all their keys in one LDS block; longer ones (the
// tokenizer's 1432-token frames, long time windows) are cut into key blocks
// of at most 320.
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
// Two kernels, each keeping one side of the problem stationary in registers
// so that no sum crosses waves (no atomics; bitwise deterministic; the split
// last round above adds its two halves in a fixed order):
//
//  dkv kernel (key-parallel, launched first): each wave owns 16-key tiles
//             of one problem and keeps their dK^T, dV^T accumulators and K, V
//             operands in registers; the problem's query rows stream through
//             LDS in 32-row chunks (double-buffered, prefetched into registers
//             one chunk ahead): S = Q K^T and dP = dO V^T, then dV^T += dO^T P
//             and dK^T += Q^T dS on MFMA, with the Q^T and dO^T operands read
//             straight from the row-major chunk by transposing LDS reads.
//             Staging a chunk also forms its rows' Delta from dO and O.
//             When the problem's keys fit one block (at most 320: every
//             dynamics shape), the kernel also forms dQ: each chunk's dS
//             goes to LDS, and during the next chunk that chunk's
//             dQ^T = K^T dS^T is formed from it and an LDS copy of K: by
//             every wave as one 16 x 16 block, or, for blocks of more than
//             256 keys (three tile slots), by two dedicated waves as two
//             32 x 32 blocks on v_mfma_f32_32x32x16_bf16 (half the operand
//             reads per product), those two waves keeping one key tile each.
//             The dq kernel is then not launched.  In that three-slot
//             layout waves 0..3 stage whole chunks and waves 4..7 run at
//             wave priority 1, so both waves of a SIMD reach the chunk
//             barrier together.  One workgroup per problem and CU makes the
//             problems pass through the device in rounds; a last round at
//             most half full runs as two workgroups per problem (query rows
//             split), whose fp32 dK, dV partials a small kernel sums in a
//             fixed order.
//  dq kernel  (query-parallel, laid out like the forward; longer problems
//             only): a workgroup holds K, V and K^T of one (unit, KV head)
//             problem's key block in LDS; each wave owns 32 query rows
//             (position x head-in-group) and sweeps the visible keys in
//             32-key steps: S^T = K Q^T and dP^T = V dO^T on MFMA (every lane
//             holds one query column), P^T and dS^T on VALU, dQ^T += K^T dS^T
//             on MFMA.  Delta comes from the workspace the dkv kernel wrote.
//
// Key steps (dq, and the dQ steps of the dkv kernel) and query chunks (dkv)
// that the causal / window ranges make invisible are never visited.  For
// long problems the split costs two more matmul passes (S and dP are formed
// in both kernels) in exchange for no cross-workgroup sum of dQ.
//
// Windowed time attention over more than 320 frames avoids the split: the
// fused dkv kernel runs each problem as segments of R query positions (R +
// W - 1 <= 320, R * G a whole number of 32-row chunks).  A segment's rows see
// only the keys [s R - W + 1, (s + 1) R), which fit one block, so it forms
// their dQ completely; its dK, dV cover keys that neighbouring segments'
// rows see too, so they go out as fp32 partials and the segment reduce
// kernel adds, per key, the partials of the segments that hold it in
// segment order (deterministic).
#include <algorithm>
#include <mutex>

#include "bca_device.h"
#include "bca_kernels.h"

namespace bca {

namespace {

constexpr int KMAX = kBwdKeyBlock;  // 320

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
  float* delta;  // workspace, (B, T, N, Hq) fp32
  int T, N, Hq, Hkv, G, L, units, rows;
  int window, agent_begin, agent_count;
  float scale, scale_log2, inv_g;
  int splits, rows_per_split;  // dq kernel
  int kvb, kbl;                // dkv kernel: key blocks per problem, keys per block
  int poison;                  // debug: NaN-fill LDS before staging
  // fused backward, last round split: problems from split_base on run as
  // two workgroups each, rows of chunks [.., split_chunk) and [split_chunk,
  // ..), whose fp32 dK, dV partials (split_keys keys x 128 per half) go to
  // part and are summed by the reduce kernel
  int split_base, split_chunk, split_keys;
  float* part;
  // fused backward of windowed time attention over more than one key block:
  // each problem runs as nseg workgroups, segment s owning the query rows of
  // positions [s * seg_pos, (s + 1) * seg_pos) and the keys they see,
  // [s * seg_pos - window + 1, (s + 1) * seg_pos) (at most seg_keys); its
  // fp32 dK, dV partials (seg_keys keys x 128) go to part and the segment
  // reduce kernel sums them (0 segments: not this path)
  int nseg, seg_pos, seg_keys;
};

// ------------------------------------------------------------- dq kernel

constexpr int DQ_W = 12;   // waves per workgroup
constexpr int DQ_QC = 32;  // query rows per wave and chunk

__device__ __forceinline__ int krow_off(int key, int chunk) {  // [KMAX][64], 16B chunks xor-swizzled
  return key * 64 + ((chunk ^ (key & 7)) << 3);
}
// K^T is stored with keys permuted inside each group of 32 so that the 8 keys
// a lane feeds to one MFMA are contiguous: key 32a + 16h + 4g + j sits at
// position 32a + 8g + 4h + j.
__device__ __forceinline__ int kperm(int key) {
  return (key & ~31) | (((key >> 2) & 3) << 3) | (((key >> 4) & 1) << 2) | (key & 3);
}
__device__ __forceinline__ int kt_off(int d, int pos) {  // [64][KMAX]
  return d * KMAX + ((((pos >> 3) ^ (d & 7))) << 3) + (pos & 7);
}

struct DqSmem {
  bf16 K[KMAX * 64];
  bf16 V[KMAX * 64];
  bf16 KT[64 * KMAX];
};

template <int OP>
__global__ __attribute__((amdgpu_flat_work_group_size(DQ_W * 64, DQ_W * 64), amdgpu_waves_per_eu(3, 3)))
void attn_bwd_dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) DqSmem sm;
  constexpr int NT = DQ_W * 64;
  if (p.poison) {
    poison_lds(&sm, sizeof(sm), threadIdx.x, NT);
    __syncthreads();
  }

  int ug, split;
  xcd_remap(blockIdx.x, p.units * p.Hkv, p.splits, ug, split);
  const int u = ug / p.Hkv, g = ug - (ug / p.Hkv) * p.Hkv;
  const UnitGeom gq = unit_geom(OP, u, p.T, p.N, p.Hq, 64);
  const UnitGeom gk = unit_geom(OP, u, p.T, p.N, p.Hkv, 64);
  const UnitGeom gl = unit_geom(OP, u, p.T, p.N, p.Hq, 1);
  const MaskDesc md{OP, p.L, p.window, p.agent_begin, p.agent_count};
  const int G = p.G;
  const int64_t qhead = (int64_t)g * G * 64;
  const bf16* kbase = p.k + gk.base + g * 64;
  const bf16* vbase = p.v + gk.base + g * 64;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int li = lane & 15, lg = lane >> 4;
  const int row0 = split * p.rows_per_split;
  const int row1 = min(p.rows, row0 + p.rows_per_split);
  const int nch = (row1 - row0 + DQ_QC - 1) / DQ_QC;

  // Keys [wklo, wkhi) are all that any row of this workgroup sees; they pass
  // through LDS in blocks of up to KMAX keys (one block, staged once, for the
  // dynamics shapes), at LDS position key - key0 (rows past the block's end
  // zero-filled up to a multiple of 32).  Keys staged as padding are never
  // counted twice: a step that reaches past the block end is masked, because
  // those keys lie beyond every row's range or past L.
  int wklo, wkhi;
  key_range(md, row0 / G, (row1 - 1) / G, wklo, wkhi);
  wklo &= ~31;  // steps stay aligned to 32 keys (the extra keys are masked)
  const int nkb = (wkhi - wklo + KMAX - 1) / KMAX;
  auto stage = [&](int key0, int kn) {
    const int lp32 = (kn + 31) & ~31;
    for (int idx = tid; idx < lp32 * 8; idx += NT) {
      const int r = idx >> 3, c = idx & 7;
      const bool ok = r < kn;
      const int64_t off = (int64_t)(key0 + (ok ? r : 0)) * gk.pos_stride + c * 8;
      const bf16x8 kv = ok ? ld_global16(kbase + off) : zero8();
      const bf16x8 vv = ok ? ld_global16(vbase + off) : zero8();
      st_lds16(sm.K + krow_off(r, c), kv);
      st_lds16(sm.V + krow_off(r, c), vv);
      const int pp = kperm(r);
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.KT[kt_off(c * 8 + e, pp)] = kv[e];
    }
  };
  if (nkb == 1) {
    stage(wklo, wkhi - wklo);
    __syncthreads();
  }

  // Per chunk, this lane's query column in each of the two 16-column tiles
  // (padding columns read a real, clamped row and are never stored).
  struct ChunkIn {
    bf16x8 q[2][2], d[2][2];
    float lse[2], delta[2];
  };
  auto load_chunk = [&](int ch, ChunkIn& in) {
    const int r0c = row0 + ch * DQ_QC;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int rr = min(r0c + qt * 16 + li, row1 - 1);
      const int pos = row_pos(rr, p.inv_g);
      const int hq = rr - pos * G;
      const int64_t off = gq.base + (int64_t)pos * gq.pos_stride + qhead + hq * 64 + lg * 8;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        in.q[qt][s] = ld_global16(p.q + off + s * 32);
        in.d[qt][s] = ld_global16(p.dout + off + s * 32);
      }
      in.lse[qt] = p.lse[gl.base + (int64_t)pos * gl.pos_stride + g * G + hq];
      in.delta[qt] = p.delta[gl.base + (int64_t)pos * gl.pos_stride + g * G + hq];
    }
  };
  // one chunk per wave and pass; with several key blocks, every block is
  // staged once per pass and each wave accumulates its chunk's dQ over them
  const int passes = (nch + DQ_W - 1) / DQ_W;
  for (int pass = 0; pass < passes; ++pass) {
    const int ch = pass * DQ_W + wave;
    const bool active = ch < nch;
    const int r0 = row0 + ch * DQ_QC;
    bf16x8 qreg[2][2], dreg[2][2];
    int qpos[2], hh[2];
    bool qv[2];
    float lse2[2], dlt[2];
    f32x4 acc[4][2];
    int qlo = 0, qhi = 0, klo = 0, khi = 0;
    if (active) {
      ChunkIn nxt;
      load_chunk(ch, nxt);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int r = r0 + qt * 16 + li;
        qv[qt] = r < row1;
        const int rr = min(r, row1 - 1);
        qpos[qt] = row_pos(rr, p.inv_g);
        hh[qt] = rr - qpos[qt] * G;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          qreg[qt][s] = nxt.q[qt][s];
          dreg[qt][s] = nxt.d[qt][s];
        }
        dlt[qt] = nxt.delta[qt];
        lse2[qt] = qv[qt] ? nxt.lse[qt] * kLog2e : INFINITY;
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        acc[dt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      qlo = r0 / G;
      qhi = (min(r0 + DQ_QC, row1) - 1) / G;
      key_range(md, qlo, qhi, klo, khi);
    }
    for (int kb = 0; kb < nkb; ++kb) {
      const int key0 = wklo + kb * KMAX;
      const int kn = min(KMAX, wkhi - key0);
      if (nkb > 1) {
        __syncthreads();
        stage(key0, kn);
        __syncthreads();
      }
      if (!active) continue;
      const int lo = max(klo, key0), hi = min(khi, key0 + kn);
      if (lo >= hi) continue;
      const int st0 = (lo - key0) >> 5, st1 = (hi - key0 + 31) >> 5;
      for (int st = st0; st < st1; ++st) {
        const int kabs = key0 + st * 32;  // absolute key of the step's first row
        f32x4 sc[2][2], dp[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kr = st * 32 + h * 16 + li;
          const bf16x8 k0 = ld_lds16(sm.K + krow_off(kr, lg));
          const bf16x8 k1 = ld_lds16(sm.K + krow_off(kr, 4 + lg));
          const bf16x8 v0 = ld_lds16(sm.V + krow_off(kr, lg));
          const bf16x8 v1 = ld_lds16(sm.V + krow_off(kr, 4 + lg));
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            z = mfma16(k0, qreg[qt][0], z);
            sc[qt][h] = mfma16(k1, qreg[qt][1], z);
            // the accumulator starts at -Delta, so it ends at dP - Delta
            f32x4 y = {-dlt[qt], -dlt[qt], -dlt[qt], -dlt[qt]};
            y = mfma16(v0, dreg[qt][0], y);
            dp[qt][h] = mfma16(v1, dreg[qt][1], y);
          }
        }
        bf16x8 dsb[2];
        if (tile_all_visible(md, qlo, qhi, kabs, kabs + 32) && kabs + 32 <= key0 + kn) {
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            f32x4 d0, d1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              d0[j] = fast_exp2(__builtin_fmaf(sc[qt][0][j], p.scale_log2, -lse2[qt])) * dp[qt][0][j];
              d1[j] = fast_exp2(__builtin_fmaf(sc[qt][1][j], p.scale_log2, -lse2[qt])) * dp[qt][1][j];
            }
            dsb[qt] = pack8(d0, d1);
          }
        } else {
          const int kend = key0 + kn;
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            f32x4 d0, d1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int ka = kabs + lg * 4 + j, kc = kabs + 16 + lg * 4 + j;
              const bool vis0 = visible_op<OP>(md, qpos[qt], ka) & (ka < kend);
              const bool vis1 = visible_op<OP>(md, qpos[qt], kc) & (kc < kend);
              const float e0 = fast_exp2(__builtin_fmaf(sc[qt][0][j], p.scale_log2, -lse2[qt])) * dp[qt][0][j];
              const float e1 = fast_exp2(__builtin_fmaf(sc[qt][1][j], p.scale_log2, -lse2[qt])) * dp[qt][1][j];
              d0[j] = vis0 ? e0 : 0.f;
              d1[j] = vis1 ? e1 : 0.f;
            }
            dsb[qt] = pack8(d0, d1);
          }
        }
        // tile dt's operand row r is head dim 16 (r >> 2) + 4 dt + (r & 3),
        // so that each lane ends with dims 16 lg .. 16 lg + 15 of its row
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8 kt = ld_lds16(sm.KT + kt_off(16 * (li >> 2) + 4 * dt + (li & 3), st * 32 + lg * 8));
          acc[dt][0] = mfma16(kt, dsb[0], acc[dt][0]);
          acc[dt][1] = mfma16(kt, dsb[1], acc[dt][1]);
        }
      }
    }
    if (!active) continue;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      if (!qv[qt]) continue;
      bf16* dst = p.dq + gq.base + (int64_t)qpos[qt] * gq.pos_stride + qhead + hh[qt] * 64 + lg * 16;
      st_global16(dst, pack8(acc[0][qt] * p.scale, acc[1][qt] * p.scale));
      st_global16(dst + 8, pack8(acc[2][qt] * p.scale, acc[3][qt] * p.scale));
    }
  }
}

// ------------------------------------------------------------ dkv kernel

// Tile slots per wave TPW: one (16 waves, four per SIMD), two or three (8
// waves; tile = wave + waves * slot).  Waves 0..7 form dQ; with 16 waves,
// waves 8..15 stage the query chunks (with 8, every wave does both).
template <int TPW>
constexpr int kv_waves() { return TPW == 1 ? 16 : 8; }
constexpr int KV_QC = 32;  // query rows per chunk

// With the query gradient formed by waves 6 and 7 on 32x32 products (DQ32:
// one key block per problem, three tile slots), those two waves keep one key
// tile each and waves 0..5 up to three: slot 0 holds tiles 0..7 (wave w has
// tile w), slot 1 tiles 8..13 and slot 2 tiles 14..19 (waves 0..5), so a
// block of up to 320 keys is covered.  Otherwise tile = wave + waves * slot.
template <int KV_W, bool DQ32>
__device__ __forceinline__ int tile_of(int wave, int m) {
  if constexpr (DQ32) {
    if (m == 0) return wave;
    return wave < 6 ? 8 + 6 * (m - 1) + wave : 1 << 20;
  } else {
    return wave + KV_W * m;
  }
}

__device__ __forceinline__ int row_off(int row, int chunk) {  // [32][64]
  return row * 64 + ((chunk ^ (row & 7)) << 3);
}
// Offset of the 8-byte piece this lane addresses in a transposing read of
// the row-major chunk tile: rows 16*h + 4*g + (li >> 2), columns
// 16*dt + 4*(li & 3) .. +3.  Lane (li, g) then receives column 16*dt + li of
// rows 16*h + 4*g + 0..3, i.e. four of the 8 queries it feeds to one MFMA.
__device__ __forceinline__ int tr_piece_off(int h, int dt, int li, int lg) {
  const int row = 16 * h + 4 * lg + (li >> 2);
  const int col = 16 * dt + 4 * (li & 3);
  return row * 64 + ((((col >> 3) ^ (row & 7))) << 3) + (col & 7);
}

// One DPP lane move (row_mask and bank_mask all set).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

struct KvBuf {
  bf16 Q[KV_QC * 64];
  bf16 dO[KV_QC * 64];
  float lse[KV_QC];     // log2-scaled LSE of the rows (+inf for padding)
  float ndelta[KV_QC];  // -Delta of the rows
  // space attention: the LSE as agent keys see it, +inf for world rows
  // (which cannot see them), so that P of such a pair is exp2(-inf) = 0
  float lse_agent[KV_QC];
};
// the lane offsets below add 16 rows as 2048 bytes and reach dO from Q
static_assert(offsetof(KvBuf, dO) == KV_QC * 64 * 2, "KvBuf layout");

// With the query gradient formed in the same kernel (FQ), the block's K rows
// stay in LDS (row-major, zero past the end) and each chunk's dS goes to one
// of two key-major buffers [key][32 rows], read back transposed as the B
// operand of dQ^T = K^T dS^T.
template <bool FQ>
struct KvSmem {
  KvBuf sbuf[2];
};
template <>
struct KvSmem<true> {
  KvBuf sbuf[2];
  bf16 K[KMAX * 64];
  bf16 dS[2][KMAX * KV_QC];
};
// Both buffers are laid out in 8-byte pieces swizzled so that every 32-lane
// half of a read or write touches 64 distinct 4-byte banks: K's 16 pieces of
// 4 head dims per key are xored with 4 * (bit 1 and bit 3 of the key), dS's 8
// pieces of 4 rows per key with 2 * (bits 2..3 of the key).
__device__ __forceinline__ int kq_off(int key, int d) {  // [KMAX][64]
  const int m = ((key >> 1) & 1) | (((key >> 3) & 1) << 1);
  return key * 64 + (((d >> 2) ^ (m << 2)) << 2) + (d & 3);
}
__device__ __forceinline__ int ds_off(int key, int row) {  // [KMAX][32]
  return key * KV_QC + (((row >> 2) ^ (((key >> 2) & 3) << 1)) << 2) + (row & 3);
}

// One workgroup per (unit, KV head) problem and key block.  Each wave keeps
// the K and V rows of its tiles (the B operands of S and dP) and their dK^T,
// dV^T accumulators in registers for the whole kernel; only the query rows
// pass through LDS.  With three slots the two waves of a SIMD (w and w + 4)
// hold 5 of the 20 tile slots between them.
//
// Masks are tested on folded row indices r = position * G + head: a key k is
// visible to row r in time attention iff k*G <= r < (k + W)*G, and a row is
// an agent row iff agent_begin*G <= r < (agent_begin + agent_count)*G.  The
// space mask (world rows do not see agent keys) costs no per-element test:
// each chunk carries a second LSE row, +inf for world rows, which the lanes
// holding agent keys use, so P of a hidden pair is exp2(-inf) = 0 exactly.
// Keys past the end need no mask: they only feed their own (discarded) dK, dV
// columns and, with FQ, dQ through K rows that are zero in LDS.
// GC > 0: an instance for G = GC query heads per KV head (the chunk
// positions then divide by a constant instead of a runtime G).
template <int OP, int TPW, bool FQ, int GC = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(kv_waves<TPW>() * 64, kv_waves<TPW>() * 64),
                          amdgpu_waves_per_eu(kv_waves<TPW>() / 4, kv_waves<TPW>() / 4)))
void attn_bwd_dkv_kernel(BwdParams p) {
  constexpr int KV_W = kv_waves<TPW>();
  __shared__ __attribute__((aligned(16))) KvSmem<FQ> sm;
  KvBuf* sbuf = sm.sbuf;
  if (p.poison) {
    poison_lds(&sm, sizeof(sm), threadIdx.x, KV_W * 64);
    __syncthreads();
  }

  // workgroup = (problem, block of kbl keys); one block for L <= 320.  With
  // FQ, workgroups from split_base on are halves of the last problems.
  int ug, kb, half = -1, seg = -1;
  if (FQ && (int)blockIdx.x >= p.split_base) {
    const int j = (int)blockIdx.x - p.split_base;
    ug = p.split_base + (j >> 1);
    half = j & 1;
    kb = 0;
  } else if (FQ && OP == OP_TIME && p.nseg > 0) {
    // a problem's segments go to one XCD one after another (neighbouring
    // segments share most of their keys)
    xcd_remap(blockIdx.x, p.units * p.Hkv, p.nseg, ug, seg);
    kb = 0;
  } else {
    xcd_remap(blockIdx.x, p.units * p.Hkv, p.kvb, ug, kb);
  }
  const int u = ug / p.Hkv, g = ug - (ug / p.Hkv) * p.Hkv;
  const UnitGeom gq = unit_geom(OP, u, p.T, p.N, p.Hq, 64);
  const UnitGeom gk = unit_geom(OP, u, p.T, p.N, p.Hkv, 64);
  const UnitGeom gl = unit_geom(OP, u, p.T, p.N, p.Hq, 1);
  const MaskDesc md{OP, p.L, p.window, p.agent_begin, p.agent_count};
  const int G = GC > 0 ? GC : p.G;
  const int64_t qhead = (int64_t)g * G * 64;
  // position of folded row r >= 0, and r / G on the scalar unit
  auto pos_of = [&](int r) { return GC > 0 ? (int)((unsigned)r / (unsigned)GC) : row_pos(r, p.inv_g); };
  auto div_g = [&](int r) { return GC > 0 ? (int)((unsigned)r / (unsigned)GC) : r / G; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int li = lane & 15, lg = lane >> 4;
  // first key of the block and one past its last key
  const int kb0 = seg >= 0 ? max(0, seg * p.seg_pos - p.window + 1) : kb * p.kbl;
  const int kend = seg >= 0 ? min(p.L, (seg + 1) * p.seg_pos) : min(p.L, kb0 + p.kbl);
  const int nkt = (kend - kb0 + 15) >> 4;

  // K and V operands of the wave's tiles, straight from global memory
  // (keys past the end read as zero); with FQ and three tiles the K operands
  // are read from the LDS copy of K at each use instead (register pressure)
  constexpr bool KB_LDS = FQ && TPW >= 3;
  constexpr bool DQ32 = FQ && TPW == 3;
  auto tile = [&](int m) { return tile_of<KV_W, DQ32>(wave, m); };
  bf16x8 KB[KB_LDS ? 1 : TPW][2], VB[TPW][2];
  int keyG[TPW];    // time: key * G
  bool kagent[TPW];  // space: the lane's key is an agent key
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int key = kb0 + tile(m) * 16 + li;
    const bool ok = key < kend;
    const int64_t off = gk.base + (int64_t)min(key, p.L - 1) * gk.pos_stride + g * 64;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 kv = ld_global16(p.k + off + (s * 4 + lg) * 8);
      const bf16x8 vv = ld_global16(p.v + off + (s * 4 + lg) * 8);
      if constexpr (!KB_LDS) KB[m][s] = ok ? kv : zero8();
      VB[m][s] = ok ? vv : zero8();
    }
    keyG[m] = key * G;
    kagent[m] = (unsigned)(key - p.agent_begin) < (unsigned)p.agent_count;
  }
  // time: key k is visible to folded row r iff 0 <= r - k*G < winG (no
  // window: the whole sequence, so the test still rejects r < k*G)
  const unsigned winG = (unsigned)((p.window > 0 ? p.window : p.L) * G);
  const int agentG0 = p.agent_begin * G;
  const unsigned agentGn = (unsigned)(p.agent_count * G);
  // space attention: byte offset in a chunk buffer of the LSE row that this
  // lane's key of slot m reads; agent keys read the row that is +inf for
  // world rows, which applies the agent mask with no per-element test
  int lse_at[TPW];
#pragma unroll
  for (int m = 0; m < TPW; ++m)
    lse_at[m] = (int)(kagent[m] ? offsetof(KvBuf, lse_agent) : offsetof(KvBuf, lse));

  f32x4 dKT[TPW][4], dVT[TPW][4];
#pragma unroll
  for (int m = 0; m < TPW; ++m)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      dKT[m][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dVT[m][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // staging (by waves 8..15 with 16 waves, as they form no dQ; by all 8
  // otherwise): the first 256 staging threads carry Q (and LSE), the next 256
  // dO (and Delta); a piece is (row, 16-byte column chunk) of the chunk.  The
  // loads are only issued by fetch(); the LSE transform waits for stage() so
  // that no wave stalls on a global load a chunk early.  In the DQ32 layout
  // waves 0..3 stage both halves (each thread its Q and its dO piece), so
  // that the dQ waves 6, 7 stage nothing.
  constexpr bool STAGE_LOW = DQ32;
  const int stid = KV_W > 8 ? tid - 512 : tid;
  const bool carries_q = (stid & 511) < 256;
  const bool stager = KV_W > 8 ? stid >= 0 : !STAGE_LOW || tid < 256;
  const int srow = (tid & 255) >> 3, sch = tid & 7;
  bf16x8 pre = zero8(), pre_o = zero8(), pre_q = zero8();
  float pre_s = 0.f;
  bool pre_valid = false, pre_agent = false;
  int64_t pre_lo = 0;
  auto fetch = [&](int c) {
    if (!stager) return;
    // padding rows read a real (clamped) row; their LSE of +inf zeroes P
    const int r = c * KV_QC + srow;
    pre_valid = r < p.rows;
    if constexpr (OP == OP_SPACE) pre_agent = (unsigned)(r - agentG0) < agentGn;
    const int rr = min(r, p.rows - 1);
    const int pos = pos_of(rr);
    const int hh = rr - pos * G;
    const int64_t off = gq.base + (int64_t)pos * gq.pos_stride + qhead + hh * 64 + sch * 8;
    const int64_t lo = gl.base + (int64_t)pos * gl.pos_stride + g * G + hh;
    if constexpr (STAGE_LOW) {
      pre_q = ld_global16(p.q + off);
      pre_s = p.lse[lo];
      pre = ld_global16(p.dout + off);
      pre_o = ld_global16(p.o + off);
    } else {
      // (the base chosen per wave, a scalar select: the same as carries_q)
      pre = ld_global16((((wave & 7) < 4) ? p.q : p.dout) + off);
      if (carries_q)
        pre_s = p.lse[lo];
      else
        pre_o = ld_global16(p.o + off);
    }
    pre_lo = lo;
  };
  // Delta = rowsum(dO * O) is formed here, from the 8 pieces of a row held by
  // 8 adjacent threads; the chunk buffer keeps -Delta, and without FQ it also
  // goes to the workspace for the dq kernel (which runs after this one), where
  // workgroups whose chunk ranges overlap write the same bits
  auto stage = [&](KvBuf& b) {
    if (!stager) return;
    if constexpr (STAGE_LOW) {
      st_lds16(b.Q + row_off(srow, sch), pre_q);
      st_lds16(b.dO + row_off(srow, sch), pre);
    } else {
      st_lds16((carries_q ? b.Q : b.dO) + row_off(srow, sch), pre);
    }
    if (STAGE_LOW || carries_q) {
      if (sch == 0) {
        const float l2 = pre_valid ? pre_s * kLog2e : INFINITY;
        b.lse[srow] = l2;
        if constexpr (OP == OP_SPACE) b.lse_agent[srow] = pre_agent ? l2 : INFINITY;
      }
    }
    if (STAGE_LOW || !carries_q) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) t = __builtin_fmaf((float)pre[e], (float)pre_o[e], t);
      // sum over the 8 lanes of the row: quad swaps (1 0 3 2), (2 3 0 1),
      // then the half-row mirror pairs each quad with the other one
      t += dpp_f32<0xB1>(t);
      t += dpp_f32<0x4E>(t);
      t += dpp_f32<0x141>(t);
      if (sch == 0) {
        b.ndelta[srow] = -t;
        if (!FQ && pre_valid) p.delta[pre_lo] = t;
      }
    }
  };

  // query chunks that can see a key of the block: time attention skips the
  // rows before it and those more than the window after it
  int c_lo = 0, c_hi = (p.rows + KV_QC - 1) / KV_QC;
  if (OP == OP_TIME) {
    c_lo = (kb0 * G) / KV_QC;
    if (p.window > 0) {
      const int64_t rend = min((int64_t)p.rows, (int64_t)(kend - 1 + p.window) * G);
      c_hi = min(c_hi, (int)((rend + KV_QC - 1) / KV_QC));
    }
  }
  if (half == 0) c_hi = min(c_hi, p.split_chunk);
  if (half == 1) c_lo = max(c_lo, p.split_chunk);
  if (seg >= 0) {
    // the segment's own rows (seg_pos * G is a whole number of chunks); the
    // keys they see all lie in [kb0, kend), so their dQ is complete here
    c_lo = seg * p.seg_pos * G / KV_QC;
    c_hi = (min(p.L, (seg + 1) * p.seg_pos) * G + KV_QC - 1) / KV_QC;
  }
  const int nchunks = c_hi;

  // byte offsets of this lane's LDS reads within a chunk buffer, formed once
  // and kept in registers (the 16-row half, dO and the buffer are added as
  // constants): row-major reads of rows li (+16), column chunks s*4 + lg,
  // and the transposing reads of column slice dt
  int offQ[2], offT[4];
#pragma unroll
  for (int s = 0; s < 2; ++s) offQ[s] = row_off(li, s * 4 + lg) * 2;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) offT[dt] = tr_piece_off(0, dt, li, lg) * 2;
#pragma unroll
  for (int s = 0; s < 2; ++s) asm volatile("" : "+v"(offQ[s]));
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) asm volatile("" : "+v"(offT[dt]));
  // FQ: the block's K rows into LDS, rows up to a multiple of 32 keys
  // (zero past the end, so that dS of those keys meets zero K)
  const int nks = ((nkt * 16 + 31) >> 5) << 5;  // keys covered by the dQ steps
  if constexpr (FQ) {
    const bf16* kbase = p.k + gk.base + g * 64;
    for (int idx = tid; idx < nks * 8; idx += KV_W * 64) {
      const int r = idx >> 3, ch = idx & 7;
      const bool ok = kb0 + r < kend;
      const bf16x8 kv = ok ? ld_global16(kbase + (int64_t)(kb0 + r) * gk.pos_stride + ch * 8) : zero8();
      st_lds16(sm.K + kq_off(r, ch * 8), kv);
    }
  }
  // FQ, dQ of chunk cq from its dS buffer, over the 32-key steps that hold
  // the chunk's visible keys: with 8 waves, wave w forms the 16 x 16 block
  // of dQ^T for head-dim slice w & 3 and row half w >> 2; with 16, waves 0..3
  // form two such blocks each, for row half w >> 1 and the 32 dims from 32 (w
  // & 1), whose operand rows are permuted (block t, row r: dim 32 (w & 1) + 8
  // (r >> 2) + 4 t + (r & 3)) so that each lane ends with 8 consecutive dims
  // of its row and stores them as one 16-byte piece
  // Lane offsets (elements) into the swizzled K and dS buffers, formed once:
  // the swizzles depend only on key bits 1..3, so moving by 16 keys (a tile)
  // or 32 (a dQ step) adds a constant.  dQ reads: key 8 lg + (li >> 2) (+4)
  // of a step, head dims (w & 3)*16 + 4 (li & 3), rows (w >> 2)*16 + 4 (li & 3);
  // dS writes: key li of a tile, rows 16 qt + 4 lg; K operand reads (three
  // slots): key li of a tile, head dims 8 (4 s + lg).
  int oK[2] = {0, 0}, oD[2] = {0, 0}, oW[2] = {0, 0}, oB[2] = {0, 0};
  if constexpr (FQ) {
    const int kq = 8 * lg + (li >> 2);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if constexpr (KV_W > 8) {
        // block 1's dims are block 0's + 4, which in kq_off's swizzle (even
        // 4-dim piece index, xor on bits 2..3 of it) is 4 elements further
        oK[e] = kq_off(kq + 4 * e, 32 * (wave & 1) + 8 * (li & 3));
        oD[e] = ds_off(kq + 4 * e, ((wave >> 1) & 1) * 16 + 4 * (li & 3));
      } else {
        oK[e] = kq_off(kq + 4 * e, (wave & 3) * 16 + 4 * (li & 3));
        oD[e] = ds_off(kq + 4 * e, (wave >> 2) * 16 + 4 * (li & 3));
      }
      oW[e] = ds_off(li, e * 16 + 4 * lg);
      oB[e] = kq_off(li, (4 * e + lg) * 8);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) asm volatile("" : "+v"(oK[e]), "+v"(oD[e]), "+v"(oW[e]), "+v"(oB[e]));
  }
  auto dq_phase = [&](int cq) {
    if constexpr (FQ) {
      if (wave >= (KV_W > 8 ? 4 : 8)) return;
      const int r0q = cq * KV_QC;
      const int qlo = div_g(r0q), qhi = div_g(min(r0q + KV_QC, p.rows) - 1);
      int klo, khi;
      key_range(md, qlo, qhi, klo, khi);
      const int st0 = max(klo - kb0, 0) >> 5, st1 = (min(khi, kend) - kb0 + 31) >> 5;
      const bf16* dsb = sm.dS[cq & 1];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      for (int st = st0; st < st1; ++st) {
        // four head-dim columns of K and four rows of dS per lane and read
        const bf16* kst = sm.K + st * 32 * 64;
        const bf16* dst_ = dsb + st * 32 * KV_QC;
        const bf16x8 a = join8(ld_lds_tr4(kst + oK[0]), ld_lds_tr4(kst + oK[1]));
        const bf16x8 bq = join8(ld_lds_tr4(dst_ + oD[0]), ld_lds_tr4(dst_ + oD[1]));
        acc = mfma16(a, bq, acc);
        if constexpr (KV_W > 8) {
          const bf16x8 a1 = join8(ld_lds_tr4(kst + oK[0] + 4), ld_lds_tr4(kst + oK[1] + 4));
          acc1 = mfma16(a1, bq, acc1);
        }
      }
      if constexpr (KV_W > 8) {
        // lane (li, lg): row (w >> 1)*16 + li of the chunk, dims 32 (w & 1) + 8 lg .. +7
        const int r = r0q + ((wave >> 1) & 1) * 16 + li;
        if (r < p.rows) {
          const int pos = pos_of(r);
          const int hh = r - pos * G;
          bf16* dst = p.dq + gq.base + (int64_t)pos * gq.pos_stride + qhead + hh * 64 + 32 * (wave & 1) + 8 * lg;
          st_global16(dst, pack8(acc * p.scale, acc1 * p.scale));
        }
      } else {
        // lane (li, lg): row (w >> 2)*16 + li of the chunk, dims (w & 3)*16 + 4 lg ..
        const int r = r0q + (wave >> 2) * 16 + li;
        if (r < p.rows) {
          const int pos = pos_of(r);
          const int hh = r - pos * G;
          bf16* dst = p.dq + gq.base + (int64_t)pos * gq.pos_stride + qhead + hh * 64 + (wave & 3) * 16 + lg * 4;
          *reinterpret_cast<u32x2*>(dst) = __builtin_bit_cast(u32x2, pack4(acc * p.scale));
        }
      }
    }
  };
  // DQ32: wave 6 + a forms the 32 x 32 block of the chunk's dQ^T for head
  // dims 32a .. 32a + 31 (all 32 rows) on v_mfma_f32_32x32x16_bf16, over
  // 16-key steps.  Operand layout: lane l holds row l % 32 of A and column
  // l % 32 of B (query row) for contraction indices (keys) 8 (l / 32) ..
  // +7, each as two transposing reads of 4 keys.  A's row rho is head dim
  // 32a + 16 ((rho >> 2) & 1) + 4 (rho >> 3) + (rho & 3), so that the output
  // lane l, which holds rows 8 q + 4 (l / 32) + j (q, j < 4), ends with the
  // 16 consecutive dims 32a + 16 (l / 32) .. +15 of query row l % 32 (two
  // 16-byte stores).  In the transposing reads, lane i of a 16-lane group
  // receives the dim that the lanes with i' & 3 == i >> 2 address, plus
  // i & 3.
  int oK32[2] = {0, 0}, oD32[2] = {0, 0};
  if constexpr (DQ32) {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int kq = 8 * (g16 >> 1) + (i16 >> 2);  // key of this lane's piece (+4 for the second)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      oK32[e] = kq_off(kq + 4 * e, 32 * (wave & 1) + 8 * (g16 & 1) + 16 * (i16 & 1) + 4 * ((i16 >> 1) & 1));
      oD32[e] = ds_off(kq + 4 * e, 16 * (g16 & 1) + 4 * (i16 & 3));
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) asm volatile("" : "+v"(oK32[e]), "+v"(oD32[e]));
  }
  auto dq_phase32 = [&](int cq) {
    if constexpr (DQ32) {
      if (wave < 6) return;
      const int r0q = cq * KV_QC;
      const int qlo = div_g(r0q), qhi = div_g(min(r0q + KV_QC, p.rows) - 1);
      int klo, khi;
      key_range(md, qlo, qhi, klo, khi);
      const int s0 = max(klo - kb0, 0) >> 4, s1 = (min(khi, kend) - kb0 + 15) >> 4;
      const bf16* dsb = sm.dS[cq & 1];
      // two accumulators (even and odd steps), so that consecutive
      // products do not wait on each other
      f32x16 acc = {}, acc1 = {};
      int st = s0;
      for (; st + 1 < s1; st += 2) {
        const bf16* kst = sm.K + st * 16 * 64;
        const bf16* dst_ = dsb + st * 16 * KV_QC;
        const bf16x8 a = join8(ld_lds_tr4(kst + oK32[0]), ld_lds_tr4(kst + oK32[1]));
        const bf16x8 bq = join8(ld_lds_tr4(dst_ + oD32[0]), ld_lds_tr4(dst_ + oD32[1]));
        const bf16x8 a1 = join8(ld_lds_tr4(kst + 16 * 64 + oK32[0]), ld_lds_tr4(kst + 16 * 64 + oK32[1]));
        const bf16x8 b1 = join8(ld_lds_tr4(dst_ + 16 * KV_QC + oD32[0]), ld_lds_tr4(dst_ + 16 * KV_QC + oD32[1]));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq, acc, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc1, 0, 0, 0);
      }
      if (st < s1) {
        const bf16* kst = sm.K + st * 16 * 64;
        const bf16* dst_ = dsb + st * 16 * KV_QC;
        const bf16x8 a = join8(ld_lds_tr4(kst + oK32[0]), ld_lds_tr4(kst + oK32[1]));
        const bf16x8 bq = join8(ld_lds_tr4(dst_ + oD32[0]), ld_lds_tr4(dst_ + oD32[1]));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq, acc, 0, 0, 0);
      }
      // hipcc has left only 11 of the 12 wait states a 32x32x16 result needs
      // on the path that skips the odd step; a fixed pad covers every path
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 11" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      acc += acc1;
      const int r = r0q + (lane & 31);
      if (r < p.rows) {
        const int pos = pos_of(r);
        const int hh = r - pos * G;
        bf16* dst = p.dq + gq.base + (int64_t)pos * gq.pos_stride + qhead + hh * 64 + 32 * (wave & 1) + 16 * (lane >> 5);
        f32x4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[q] = f32x4{acc[4 * q] * p.scale, acc[4 * q + 1] * p.scale, acc[4 * q + 2] * p.scale,
                       acc[4 * q + 3] * p.scale};
        st_global16(dst, pack8(v[0], v[1]));
        st_global16(dst + 8, pack8(v[2], v[3]));
      }
    }
  };
  // DQ32: the waves that stage nothing (4..7) issue first on their SIMD, so
  // that the two waves of a SIMD (w, w + 4) reach the chunk barrier closer
  // together (measured per-wave: the older wave 0..3 otherwise ran ahead
  // and waited at the barrier while its partner finished alone)
  if constexpr (DQ32) {
    if (wave >= 4) __builtin_amdgcn_s_setprio(1);
  }
  fetch(c_lo);
  stage(sbuf[c_lo & 1]);
  if (c_lo + 1 < nchunks) fetch(c_lo + 1);
  __syncthreads();

  for (int c = c_lo; c < nchunks; ++c) {
    KvBuf& b = sbuf[c & 1];
    const char* bb = reinterpret_cast<const char*>(&b);
    const int r0 = c * KV_QC;
    const int qlo = div_g(r0);
    const int qhi = div_g(min(r0 + KV_QC, p.rows) - 1);
    bool work[TPW], edge[TPW];
    bool anyw = false;
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int t = tile(m);
      const int k0 = kb0 + t * 16, k1 = min(k0 + 16, kend);
      work[m] = t < nkt && !tile_none_visible(md, qlo, qhi, k0, k1);
      // (space attention needs no per-element mask: see lse_at)
      edge[m] = OP == OP_TIME && !tile_all_visible(md, qlo, qhi, k0, k1);
      anyw |= work[m];
    }
    bf16x8 Pb[TPW], dSb[TPW];
    if (anyw) {
      // 1. S and dP for the owned tiles, then P and dS as packed B operands;
      // both 16-row halves of the chunk go through a tile together, so that
      // each tile carries two independent MFMA / exp chains
      bf16x4 Ph[TPW][2], dSh[TPW][2];
      bf16x8 Qa[2][2], dOa[2][2];
      f32x4 lse4[2], ndl4[2];
      auto load_stats = [&](int m) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          if constexpr (OP == OP_SPACE)
            lse4[qt] = *reinterpret_cast<const f32x4*>(bb + lse_at[m] + (qt * 16 + lg * 4) * 4);
          else
            lse4[qt] = *reinterpret_cast<const f32x4*>(b.lse + qt * 16 + lg * 4);
          ndl4[qt] = *reinterpret_cast<const f32x4*>(b.ndelta + qt * 16 + lg * 4);
        }
      };
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          Qa[qt][s] = ld_lds16(reinterpret_cast<const bf16*>(bb + offQ[s] + qt * 2048));
          dOa[qt][s] = ld_lds16(reinterpret_cast<const bf16*>(bb + offQ[s] + qt * 2048 + KV_QC * 128));
        }
      }
      // one read of the statistics per chunk, or per slot: with three slots
      // (register pressure) and for space attention (each slot's LSE row)
      constexpr bool STATS_PER_TILE = TPW >= 3 || OP == OP_SPACE;
      if constexpr (!STATS_PER_TILE) load_stats(0);
      const int rb = r0 + lg * 4;  // folded row of element j of half qt: rb + 16 qt + j
#pragma unroll
      for (int m = 0; m < TPW; ++m) {
        if (!work[m]) continue;
        if constexpr (STATS_PER_TILE) {
          // read again for every slot rather than held across the loop
          asm volatile("" ::: "memory");
          load_stats(m);
        }
        f32x4 S[2], dP[2], P[2];
        bf16x8 kop[2];
        if constexpr (KB_LDS) {
          kop[0] = ld_lds16(sm.K + tile(m) * 16 * 64 + oB[0]);
          kop[1] = ld_lds16(sm.K + tile(m) * 16 * 64 + oB[1]);
        } else {
          kop[0] = KB[m][0];
          kop[1] = KB[m][1];
        }
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          S[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
          S[qt] = mfma16(Qa[qt][0], kop[0], S[qt]);
          S[qt] = mfma16(Qa[qt][1], kop[1], S[qt]);
        }
        // the accumulator starts at -Delta, so it ends at dP - Delta
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          dP[qt] = mfma16(dOa[qt][0], VB[m][0], ndl4[qt]);
          dP[qt] = mfma16(dOa[qt][1], VB[m][1], dP[qt]);
        }
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int j = 0; j < 4; ++j) P[qt][j] = fast_exp2(__builtin_fmaf(S[qt][j], p.scale_log2, -lse4[qt][j]));
        if (edge[m]) {
#pragma unroll
          for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const bool vis = (unsigned)(rb + qt * 16 + j - keyG[m]) < winG;
              P[qt][j] = vis ? P[qt][j] : 0.f;
            }
        }
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          f32x4 dS;
#pragma unroll
          for (int j = 0; j < 4; ++j) dS[j] = P[qt][j] * dP[qt][j];
          Ph[m][qt] = pack4(P[qt]);
          dSh[m][qt] = pack4(dS);
        }
      }
      for (int m = 0; m < TPW; ++m) {
        Pb[m] = join8(Ph[m][0], Ph[m][1]);
        dSb[m] = join8(dSh[m][0], dSh[m][1]);
      }
    }
    if constexpr (FQ) {
      // this chunk's dS (zero for tiles that see none of its rows), for the
      // dQ step of the next iteration; lane (li, lg) holds rows 4 lg .. +3 of
      // each half for key li of the tile
      bf16* dsw = sm.dS[c & 1];
#pragma unroll
      for (int m = 0; m < TPW; ++m) {
        const int t = tile(m);
        if (t * 16 >= nks) continue;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          u32x2 v = {0u, 0u};
          if (work[m]) {
            const u32x4 w4 = __builtin_bit_cast(u32x4, dSb[m]);
            v = qt ? u32x2{w4[2], w4[3]} : u32x2{w4[0], w4[1]};
          }
          *reinterpret_cast<u32x2*>(dsw + t * 16 * KV_QC + oW[qt]) = v;
        }
      }
    }
    // the next chunk goes into the other buffer (last read before the
    // previous barrier) while this chunk's second phase runs
    if (c + 1 < nchunks) {
      stage(sbuf[(c + 1) & 1]);
      if (c + 2 < nchunks) fetch(c + 2);
    }
    if (anyw) {
      // 2. dV^T += dO^T P and dK^T += Q^T dS; all transposed operands are
      // read first so that one LDS round trip covers the whole phase
      bf16x8 qta[4], dota[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const char* t0 = bb + offT[dt];
        qta[dt] = join8(ld_lds_tr4(reinterpret_cast<const bf16*>(t0)),
                        ld_lds_tr4(reinterpret_cast<const bf16*>(t0 + 2048)));
        dota[dt] = join8(ld_lds_tr4(reinterpret_cast<const bf16*>(t0 + KV_QC * 128)),
                         ld_lds_tr4(reinterpret_cast<const bf16*>(t0 + KV_QC * 128 + 2048)));
      }
#pragma unroll
      for (int m = 0; m < TPW; ++m) {
        if (!work[m]) continue;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          dVT[m][dt] = mfma16(dota[dt], Pb[m], dVT[m][dt]);
          dKT[m][dt] = mfma16(qta[dt], dSb[m], dKT[m][dt]);
        }
      }
    }
    // the previous chunk's dS buffer is complete (written before the last
    // barrier) and is rewritten only after the next one
    if (DQ32 && c > c_lo) dq_phase32(c - 1);
    if (FQ && !DQ32 && c > c_lo) dq_phase(c - 1);
    __syncthreads();
  }
  if (DQ32 && nchunks > c_lo) dq_phase32(nchunks - 1);
  if (FQ && !DQ32 && nchunks > c_lo) dq_phase(nchunks - 1);

  if (FQ && seg >= 0) {
    // a segment: its fp32 partials of the keys [kb0, kend), (64 dK, 64 dV) each
    float* dst = p.part + ((int64_t)ug * p.nseg + seg) * p.seg_keys * 128;
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int key = kb0 + tile(m) * 16 + li;
      if (key >= kend) continue;
      const int64_t at = (int64_t)(key - kb0) * 128;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        *reinterpret_cast<f32x4*>(dst + at + dt * 16 + lg * 4) = dKT[m][dt];
        *reinterpret_cast<f32x4*>(dst + at + 64 + dt * 16 + lg * 4) = dVT[m][dt];
      }
    }
    return;
  }
  if (FQ && half >= 0) {
    // a half problem: its fp32 partials, keys x (64 dK, 64 dV)
    float* dst = p.part + ((int64_t)(ug - p.split_base) * 2 + half) * p.split_keys * 128;
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int key = kb0 + tile(m) * 16 + li;
      if (key >= kend) continue;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        *reinterpret_cast<f32x4*>(dst + (int64_t)key * 128 + dt * 16 + lg * 4) = dKT[m][dt];
        *reinterpret_cast<f32x4*>(dst + (int64_t)key * 128 + 64 + dt * 16 + lg * 4) = dVT[m][dt];
      }
    }
    return;
  }
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int key = kb0 + tile(m) * 16 + li;
    if (key >= kend) continue;
    bf16* dkd = p.dk + gk.base + (int64_t)key * gk.pos_stride + g * 64 + lg * 4;
    bf16* dvd = p.dv + gk.base + (int64_t)key * gk.pos_stride + g * 64 + lg * 4;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      *reinterpret_cast<u32x2*>(dkd + dt * 16) = __builtin_bit_cast(u32x2, pack4(dKT[m][dt] * p.scale));
      *reinterpret_cast<u32x2*>(dvd + dt * 16) = __builtin_bit_cast(u32x2, pack4(dVT[m][dt]));
    }
  }
}

// dK, dV of the split problems: the two halves' fp32 partials summed in a
// fixed order (half 0 + half 1), scaled (dK) and rounded to bf16.  One thread
// per (split problem, key, 8 head dims of dK or of dV).
template <int OP>
__global__ __launch_bounds__(256) void attn_bwd_split_reduce_kernel(BwdParams p, int count) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per = (int64_t)p.L * 16;
  if (idx >= (int64_t)count * per) return;
  const int sp = (int)(idx / per);
  const int rem = (int)(idx - (int64_t)sp * per);
  const int key = rem >> 4, pc = rem & 15;
  const int ug = p.split_base + sp;
  const int u = ug / p.Hkv, g = ug - (ug / p.Hkv) * p.Hkv;
  const UnitGeom gk = unit_geom(OP, u, p.T, p.N, p.Hkv, 64);
  const float* a = p.part + ((int64_t)sp * 2 * p.split_keys + key) * 128 + pc * 8;
  const float* b = a + (int64_t)p.split_keys * 128;
  const float sc = pc < 8 ? p.scale : 1.0f;
  const f32x4 a0 = *reinterpret_cast<const f32x4*>(a), a1 = *reinterpret_cast<const f32x4*>(a + 4);
  const f32x4 b0 = *reinterpret_cast<const f32x4*>(b), b1 = *reinterpret_cast<const f32x4*>(b + 4);
  bf16* dst = (pc < 8 ? p.dk : p.dv) + gk.base + (int64_t)key * gk.pos_stride + g * 64 + (pc & 7) * 8;
  st_global16(dst, pack8((a0 + b0) * sc, (a1 + b1) * sc));
}

// dK, dV of the segmented time backward: for each key, the fp32 partials of
// the segments whose key range holds it (segments key / seg_pos .. (key +
// window - 1) / seg_pos) summed in segment order, scaled (dK) and rounded to
// bf16.  One thread per (problem, key, 8 head dims of dK or of dV).
__global__ __launch_bounds__(256) void attn_bwd_seg_reduce_kernel(BwdParams p) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per = (int64_t)p.L * 16;
  if (idx >= (int64_t)p.units * p.Hkv * per) return;
  const int ug = (int)(idx / per);
  const int rem = (int)(idx - (int64_t)ug * per);
  const int key = rem >> 4, pc = rem & 15;
  const int u = ug / p.Hkv, g = ug - (ug / p.Hkv) * p.Hkv;
  const UnitGeom gk = unit_geom(OP_TIME, u, p.T, p.N, p.Hkv, 64);
  const int s0 = key / p.seg_pos, s1 = min(p.nseg - 1, (key + p.window - 1) / p.seg_pos);
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  for (int sg = s0; sg <= s1; ++sg) {
    const int kb0 = max(0, sg * p.seg_pos - p.window + 1);
    const float* src = p.part + (((int64_t)ug * p.nseg + sg) * p.seg_keys + (key - kb0)) * 128 + pc * 8;
    a0 += *reinterpret_cast<const f32x4*>(src);
    a1 += *reinterpret_cast<const f32x4*>(src + 4);
  }
  const float sc = pc < 8 ? p.scale : 1.0f;
  bf16* dst = (pc < 8 ? p.dk : p.dv) + gk.base + (int64_t)key * gk.pos_stride + g * 64 + (pc & 7) * 8;
  st_global16(dst, pack8(a0 * sc, a1 * sc));
}

// Number of compute units of the current device (0 if none).
int device_cu_count() {
  int dev = -1, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

// The fused backward runs one workgroup per problem, one per CU, so the
// problems go through the device in rounds of `cus`.  When the last round
// is at most half full, its problems are split in two by rows, so that it
// takes about half as long.  The split chunk balances an estimate of the
// chunks' cost: a fixed part and one part per key tile a chunk sees, 28 to
// 1 (timed per chunk: ~2900 cycles with one visible tile, ~4150 with 13).
struct SplitPlan {
  int base = 0x7fffffff, count = 0, chunk = 0, keys = 0;
};

SplitPlan plan_split(const AttnDims& d) {
  SplitPlan sp;
  if (!bwd_uses_mfma(d) || uses_short(d) || attended_length(d) > kBwdKeyBlock) return sp;
  const int cus = device_cu_count();
  const long problems = (long)(d.op == OP_SPACE ? (long)d.B * d.T : (long)d.B * d.N) * d.Hkv;
  if (cus <= 0 || problems <= cus) return sp;
  const long tail = problems % cus;
  if (tail == 0 || tail > cus / 2) return sp;
  const int G = d.Hq / d.Hkv, L = attended_length(d);
  const long rows = (long)L * G;
  const int chunks = (int)((rows + KV_QC - 1) / KV_QC);
  const int nkt = (L + 15) / 16;
  if (chunks < 2) return sp;
  // key tiles a chunk sees: time attention, the tiles holding keys in
  // [qlo - W + 1, qhi]; space attention, all of them
  auto cost = [&](int c) -> long {
    if (d.op != OP_TIME) return 28 + nkt;
    const long qlo = (long)c * KV_QC / G;
    const long qhi = (std::min<long>((long)c * KV_QC + KV_QC, rows) - 1) / G;
    const long klo = d.window > 0 ? std::max<long>(0, qlo - d.window + 1) : 0;
    const long t0 = klo / 16, t1 = std::min<long>(nkt - 1, qhi / 16);
    return 28 + std::max<long>(0, t1 - t0 + 1);
  };
  long total = 0;
  for (int c = 0; c < chunks; ++c) total += cost(c);
  long acc = 0, best_gap = -1;
  int best = 1;
  for (int c = 1; c < chunks; ++c) {
    acc += cost(c - 1);
    const long gap = std::max(acc, total - acc);
    if (best_gap < 0 || gap < best_gap) {
      best_gap = gap;
      best = c;
    }
  }
  sp.base = (int)(problems - tail);
  sp.count = (int)tail;
  sp.chunk = best;
  sp.keys = nkt * 16;
  return sp;
}

}  // namespace

size_t bwd_split_bytes(const AttnDims& d) {
  const SplitPlan sp = plan_split(d);
  return (size_t)sp.count * 2 * sp.keys * 128 * sizeof(float);
}

// Windowed time attention longer than one key block: the fused backward
// runs each problem as segments of seg_pos query positions, whose rows see
// at most seg_pos + W - 1 <= 320 keys, so that S and dP are formed once (the
// two-kernel path forms them in both kernels) and only the dK, dV partials
// of overlapping key ranges are summed afterwards.  seg_pos * G must be a
// whole number of 32-row chunks (so that no chunk is shared by two
// segments); segments shorter than kMinSegPos positions are not worth it
// (their key ranges overlap too much): the two-kernel path is used then.
constexpr int kMinSegPos = 128;

struct SegPlan {
  int nseg = 0, pos = 0, keys = 0;
};

SegPlan plan_segments(const AttnDims& d) {
  SegPlan sp;
  if (d.op != OP_TIME || d.window <= 0 || d.no_seg || !bwd_uses_mfma(d) || uses_short(d)) return sp;
  const int L = d.T, W = d.window, G = d.Hq / d.Hkv;
  if (L <= kBwdKeyBlock) return sp;
  int gcd = G, b = KV_QC;
  while (b) {
    const int t = gcd % b;
    gcd = b;
    b = t;
  }
  const int unit = KV_QC / gcd;  // positions per whole number of chunks
  const int R = ((kBwdKeyBlock - W + 1) / unit) * unit;
  if (R < kMinSegPos || R >= L) return sp;
  sp.pos = R;
  sp.nseg = (L + R - 1) / R;
  sp.keys = ((std::min(L, R + W - 1) + 15) / 16) * 16;
  return sp;
}

size_t bwd_seg_bytes(const AttnDims& d) {
  const SegPlan sp = plan_segments(d);
  return (size_t)d.B * d.N * d.Hkv * sp.nseg * sp.keys * 128 * sizeof(float);
}

size_t bwd_bf16_workspace_bytes(const AttnDims& d) {
  const size_t seg = bwd_seg_bytes(d);
  return seg > 0 ? seg : (size_t)d.B * d.T * d.N * d.Hq * sizeof(float);
}

// ------------------------------------------------- static scratch (no-alloc)

// Device memory of the no-allocation backward: the Delta workspace lives in
// this file-scope array instead of a caller's buffer.  Each GPU the library
// runs on holds its own copy until the process ends.  In host code the
// array's name is only a stand-in; its device address on the current device
// comes from hipGetSymbolAddress, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_attn_bwd_bf16(const AttnDims& d, const void* q, const void* k, const void* v,
                                const void* o, const float* lse, const void* dout, void* dq,
                                void* dk, void* dv, void* workspace, hipStream_t stream) {
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
  p.delta = static_cast<float*>(workspace);
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
  p.inv_g = 1.0f / (float)p.G;
  p.poison = d.poison;
  if (p.G > 256 || (long)p.rows >= (1L << 21)) return hipErrorInvalidValue;
  const long problems = (long)p.units * p.Hkv;
  p.split_base = 0x7fffffff;
  p.split_chunk = p.split_keys = 0;
  p.nseg = p.seg_pos = p.seg_keys = 0;

  // windowed time attention longer than one key block: the fused kernel
  // (three tile slots, dQ formed in it) per segment, then the partials' sum
  const SegPlan sg = plan_segments(d);
  if (sg.nseg > 0) {
    if (!workspace) return hipErrorInvalidValue;
    p.nseg = sg.nseg;
    p.seg_pos = sg.pos;
    p.seg_keys = sg.keys;
    p.kvb = 1;
    p.kbl = sg.keys;
    p.part = static_cast<float*>(workspace);
    const long grid = problems * sg.nseg;
    const long red = (problems * p.L * 16 + 255) / 256;
    if (grid > 0x7fffffff || red > 0x7fffffff) return hipErrorInvalidValue;
    if (p.G == 10)  // the dynamics model's 30 query heads over 3
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<OP_TIME, 3, true, 10>), dim3((unsigned)grid),
                         dim3(kv_waves<3>() * 64), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<OP_TIME, 3, true>), dim3((unsigned)grid),
                         dim3(kv_waves<3>() * 64), 0, stream, p);
    hipLaunchKernelGGL(attn_bwd_seg_reduce_kernel, dim3((unsigned)red), dim3(256), 0, stream, p);
    return hipGetLastError();
  }

  // dq kernel: one workgroup per CU (LDS), rows split so the grid covers the
  // CUs a few times over
  const int chunks = (p.rows + DQ_QC - 1) / DQ_QC;
  int splits = (int)((6 * 256 + problems - 1) / problems);
  splits = max(1, min(splits, (chunks + DQ_W - 1) / DQ_W));
  int per = (chunks + splits - 1) / splits;
  per = ((per + DQ_W - 1) / DQ_W) * DQ_W;
  // Windowed time attention over many frames: fewer rows per workgroup, so
  // that the keys a workgroup sees fit one LDS block (otherwise every pass
  // restages all its blocks).
  if (d.op == OP_TIME && p.window > 0)
    while (per > DQ_W && time_wg_key_span(p.L, p.G, p.window, (long)per * DQ_QC) > KMAX) per -= DQ_W;
  p.rows_per_split = per * DQ_QC;
  p.splits = (p.rows + p.rows_per_split - 1) / p.rows_per_split;
  const long g1 = problems * p.splits;
  // dkv kernel: one workgroup per problem and block of at most 320 keys,
  // blocks of equal size in whole tiles
  p.kvb = (p.L + KMAX - 1) / KMAX;
  p.kbl = (((p.L + p.kvb - 1) / p.kvb) + 15) & ~15;
  // one key block: the last round's problems may run as two halves each,
  // their dK, dV partials in the workspace (sized by bwd_split_bytes)
  const SplitPlan sp = p.kvb == 1 ? plan_split(d) : SplitPlan{};
  p.split_base = sp.base;
  p.split_chunk = sp.chunk;
  p.split_keys = sp.keys;
  p.part = static_cast<float*>(workspace);
  if (sp.count > 0 && !workspace) return hipErrorInvalidValue;
  const long g2 = problems * p.kvb + sp.count;
  if (g1 > 0x7fffffff || g2 > 0x7fffffff) return hipErrorInvalidValue;

  // Waves and tile slots per key block (measured): the fused time backward
  // with blocks of up to 256 keys, 16 waves of one tile (four per SIMD; space
  // attention's agent-mask state does not fit their 128 registers); other
  // blocks of up to 256 keys, 8 waves of two; up to 320, 8 waves of three.
  // One key block per problem: the dkv kernel forms dQ as well (from each
  // chunk's dS, which it holds in LDS), and the dq kernel is not launched.
  const bool fq = p.kvb == 1;
  const int tpw = p.kbl > 16 * 16 ? 3 : (d.op == OP_TIME && fq) ? 1 : 2;
  const dim3 g2d((unsigned)g2);
  const dim3 bw(kv_waves<1>() * 64), b8(kv_waves<3>() * 64);
  if (d.op == OP_SPACE) {
    if (fq && tpw == 2)
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<OP_SPACE, 2, true>), g2d, b8, 0, stream, p);
    else if (fq && p.G == 10)
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<OP_SPACE, 3, true, 10>), g2d, b8, 0, stream, p);
    else if (fq)
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<OP_SPACE, 3, true>), g2d, b8, 0, stream, p);
    else if (tpw == 2)
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<OP_SPACE, 2, false>), g2d, b8, 0, stream, p);
    else
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<OP_SPACE, 3, false>), g2d, b8, 0, stream, p);
    if (!fq) hipLaunchKernelGGL(attn_bwd_dq_kernel<OP_SPACE>, dim3((unsigned)g1), dim3(DQ_W * 64), 0, stream, p);
    if (sp.count > 0)
      hipLaunchKernelGGL(attn_bwd_split_reduce_kernel<OP_SPACE>, dim3((unsigned)((sp.count * (long)p.L * 16 + 255) / 256)),
                         dim3(256), 0, stream, p, sp.count);
  } else {
    if (tpw == 1 && p.G == 10)  // the dynamics model's 30 query heads over 3
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<OP_TIME, 1, true, 10>), g2d, bw, 0, stream, p);
    else if (tpw == 1)
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<OP_TIME, 1, true>), g2d, bw, 0, stream, p);
    else if (fq && p.G == 10)
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<OP_TIME, 3, true, 10>), g2d, b8, 0, stream, p);
    else if (fq)
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<OP_TIME, 3, true>), g2d, b8, 0, stream, p);
    else if (tpw == 2)
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<OP_TIME, 2, false>), g2d, b8, 0, stream, p);
    else
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<OP_TIME, 3, false>), g2d, b8, 0, stream, p);
    if (!fq) hipLaunchKernelGGL(attn_bwd_dq_kernel<OP_TIME>, dim3((unsigned)g1), dim3(DQ_W * 64), 0, stream, p);
    if (sp.count > 0)
      hipLaunchKernelGGL(attn_bwd_split_reduce_kernel<OP_TIME>, dim3((unsigned)((sp.count * (long)p.L * 16 + 255) / 256)),
                         dim3(256), 0, stream, p, sp.count);
  }
  return hipGetLastError();
}

}  // namespace bca
