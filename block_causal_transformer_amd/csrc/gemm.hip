// The projections on either side of attention, bf16 on gfx950 MFMA.
//
// Open Dreamer articles (pro.edgex.exchange, fr-FR edition): section
// "Configuration d'entraînement" (d_model 1920, 30 query heads over 3 KV
// heads of width 64) and section "Ingénierie de la stabilité", item 3
// (parameters in fp32, bf16 for most matmul activations and the attention
// inputs, fp32 for normalization layers).  The norm before the QKV projection
// is an RMS norm with an fp32 gain; weights are bf16, stored (out_features,
// in_features).  The normalized rows are never stored: the gain goes into a
// bf16 copy of the weights and each row's fp32 rstd scales its fp32 sums.
//
//  rstd_rows_kernel: one wave per token row: fp32 sum of squares,
//      rstd = 1/sqrt(mean + eps).
//  fold_gain_kernel: wg = bf16(w * gain) (the gain along the K dimension).
//  gemm_nt_kernel: C = A B^T for A (M, K) and B (N, K), both K-contiguous,
//      fp32 accumulation, bf16 results.  A 128 x 128 output tile per
//      workgroup of 4 waves (64 x 64 each), K in steps of 64 through
//      double-buffered LDS (one barrier per step, the next step's tiles
//      loaded into registers while the current one multiplies).  Each MFMA
//      forms a tile of C^T (B rows as its A operand) so a lane ends with 4
//      consecutive columns of one row: one 8-byte store.  Any M, N, K % 8.
//  gemm256_kernel: the same product with 256 x 256 tiles (256 x 192 when N
//      is a multiple of 192 but not of 256), one wave per SIMD
//      holding a 128 x 128 tile in the accumulation registers, K in steps of
//      64 through two LDS buffers filled by direct-to-LDS loads (no staging
//      registers), each refilled at mid-step, a step and a half ahead of its
//      use.  For M % 8 == N % 8 == 0, K % 64 == 0 (the projections of the
//      1920-wide layers); it halves the LDS operand traffic per MFMA.
//  Epilogues (both kernels): the QKV split (columns [0, nq) to Q, then K,
//      then V, each row-major, which is the (B,T,N,H,D) layout of the
//      attention inputs) with each row scaled by its rstd, and the residual
//      add.  gemm256_kernel passes its
//      results through LDS (16 rows per wave at a time) so that every lane
//      stores 16 contiguous bytes and a wave's lanes run along its rows, and
//      issues all of its residual loads before the first store.
#include "bca_device.h"
#include "bca_kernels.h"

namespace bca {

namespace {

constexpr int GBM = 128, GBN = 128, GBK = 64;
constexpr int GW = 4;  // waves per workgroup
constexpr int GBM2 = 256, GBN2 = 256;  // gemm256_kernel: 2 x 2 waves of 128 x 128
constexpr int WT = 8;                  // its 16-wide MFMA tiles per wave along m and n

struct GemmParams {
  const bf16* a;  // (M, K)
  const bf16* b;  // (N, K)
  int64_t M;
  int N, K;
  // epilogue 0: columns [0, nq) -> out0 (ld nq), [nq, nq+nkv) -> out1,
  // [nq+nkv, N) -> out2 (ld nkv).  epilogue 1: out0 (ld N) = C (+ residual)
  bf16* out0;
  bf16* out1;
  bf16* out2;
  const bf16* residual;
  int nq, nkv;
  int mtiles, ntiles;
  // epilogue 0 (QKV after the RMS norm): each row of C is scaled by its rstd
  const float* rstd_in;
};

__device__ __forceinline__ int tile_off(int row, int chunk) {  // [rows][64] bf16, 16B chunks xor-swizzled
  return row * GBK + ((chunk ^ (row & 7)) << 3);
}

// s plus the sum of squares of v's 8 values (fp32, by bf16 pairs: each
// square is exact in fp32)
__device__ __forceinline__ float sumsq8(const bf16x8& v, float s) {
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), __builtin_shufflevector(v, v, 0, 1), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), __builtin_shufflevector(v, v, 2, 3), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), __builtin_shufflevector(v, v, 4, 5), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), __builtin_shufflevector(v, v, 6, 7), s, false);
  return s;
}

// Stores C[m][n .. n+3] (fp32 c) through epilogue EPI; nothing past M or N.
template <int EPI>
__device__ __forceinline__ void store4(const GemmParams& p, int64_t m, int n, f32x4 c) {
  if (m >= p.M || n >= p.N) return;
  if (EPI == 0) {
    c *= p.rstd_in[m];
    bf16* dst;
    if (n < p.nq)
      dst = p.out0 + m * p.nq + n;
    else if (n < p.nq + p.nkv)
      dst = p.out1 + m * p.nkv + (n - p.nq);
    else
      dst = p.out2 + m * p.nkv + (n - p.nq - p.nkv);
    *reinterpret_cast<u32x2*>(dst) = __builtin_bit_cast(u32x2, pack4(c));
  } else {
    bf16* dst = p.out0 + m * p.N + n;
    if (p.residual) {
      const bf16x4 r = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(p.residual + m * p.N + n));
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] += (float)r[e];
    }
    *reinterpret_cast<u32x2*>(dst) = __builtin_bit_cast(u32x2, pack4(c));
  }
}

// Stores C[m][n .. n+7] (fp32 a, b) through epilogue EPI as one 16-byte
// store; nothing past M or N (N and the QKV split points are multiples of 8).
// Epilogue 0 scales the row by its rstd.
template <int EPI>
__device__ __forceinline__ void store8(const GemmParams& p, int64_t m, int n, f32x4 a, f32x4 b) {
  if (m >= p.M || n >= p.N) return;
  bf16* dst;
  if (EPI == 0) {
    const float rs = p.rstd_in[m];
    a *= rs;
    b *= rs;
    if (n < p.nq)
      dst = p.out0 + m * p.nq + n;
    else if (n < p.nq + p.nkv)
      dst = p.out1 + m * p.nkv + (n - p.nq);
    else
      dst = p.out2 + m * p.nkv + (n - p.nq - p.nkv);
  } else {
    dst = p.out0 + m * p.N + n;
    if (p.residual) {
      const bf16x8 r = ld_global16(p.residual + m * p.N + n);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] += (float)r[e];
        b[e] += (float)r[4 + e];
      }
    }
  }
  st_global16(dst, pack8(a, b));
}

// store8 for epilogue 1 with the residual piece already loaded (r)
__device__ __forceinline__ void store8r(const GemmParams& p, int64_t m, int n, f32x4 a, f32x4 b,
                                        const bf16x8& r) {
  if (m >= p.M || n >= p.N) return;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] += (float)r[e];
    b[e] += (float)r[4 + e];
  }
  st_global16(p.out0 + m * p.N + n, pack8(a, b));
}

template <int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(GW * 64, GW * 64), amdgpu_waves_per_eu(2, 2)))
void gemm_nt_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) bf16 sA[2][GBM * GBK];
  __shared__ __attribute__((aligned(16))) bf16 sB[2][GBN * GBK];

  int mt, nt;
  xcd_remap(blockIdx.x, p.mtiles, p.ntiles, mt, nt);
  const int64_t m0 = (int64_t)mt * GBM;
  const int n0 = nt * GBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int li = lane & 15, lg = lane >> 4;
  const int nk = (p.K + GBK - 1) / GBK;

  // global -> register staging: thread t moves 16-byte pieces t + 256 j of
  // each tile (row = piece / 8, 16-byte column chunk = piece % 8); rows past
  // M or N read a clamped row and are never stored, columns past K read zero
  bf16x8 ga[4], gb[4];
  auto fetch = [&](int kt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int piece = tid + GW * 64 * j;
      const int row = piece >> 3, ch = piece & 7;
      const int k = kt * GBK + ch * 8;
      const bool kok = k < p.K;
      const int64_t ar = min(m0 + row, p.M - 1);
      const int br = min(n0 + row, p.N - 1);
      const bf16x8 av = ld_global16(p.a + ar * p.K + (kok ? k : 0));
      const bf16x8 bv = ld_global16(p.b + (int64_t)br * p.K + (kok ? k : 0));
      ga[j] = kok ? av : zero8();
      gb[j] = kok ? bv : zero8();
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int piece = tid + GW * 64 * j;
      const int row = piece >> 3, ch = piece & 7;
      st_lds16(sA[buf] + tile_off(row, ch), ga[j]);
      st_lds16(sB[buf] + tile_off(row, ch), gb[j]);
    }
  };

  f32x4 acc[4][4];  // [n tile][m tile] of C^T
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  fetch(0);
  stage(0);
  if (nk > 1) fetch(1);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const bf16* A = sA[kt & 1];
    const bf16* Bt = sB[kt & 1];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 bo[4], ao[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bo[t] = ld_lds16(Bt + tile_off(wn * 64 + t * 16 + li, ks * 4 + lg));
        ao[t] = ld_lds16(A + tile_off(wm * 64 + t * 16 + li, ks * 4 + lg));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(bo[i], ao[j], acc[i][j]);
    }
    // the next step's tiles go into the other buffer (last read before the
    // previous barrier), then the loads for the step after are issued
    if (kt + 1 < nk) {
      stage((kt + 1) & 1);
      if (kt + 2 < nk) fetch(kt + 2);
    }
    __syncthreads();
  }

  // lane (li, lg) of tile (i, j) holds C[m][n .. n+3] with m = row li of the
  // m tile and n = 4 lg of the n tile
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t m = m0 + wm * 64 + j * 16 + li;
#pragma unroll
    for (int i = 0; i < 4; ++i) store4<EPI>(p, m, n0 + wn * 64 + i * 16 + lg * 4, acc[i][j]);
  }
}

// 256 x (32 WTN) output tile per workgroup of 4 waves, one wave per SIMD:
// each wave's 128 x 16 WTN tile keeps 8 WTN accumulators (up to all 256
// accumulation registers) and reads 8 + WTN LDS fragments per 8 WTN MFMAs.
// WTN = 8 (256 columns) in general; WTN = 6 (192 columns) when N is a
// multiple of 192 but not of 256 (the 1920-wide output projection: 10 full
// column tiles instead of 7.5).  K moves
// in steps of 64 through two 64 KB LDS buffers filled by direct-to-LDS loads.
// All LDS reads of a step are issued during its first half, so the buffer is
// handed back at mid-step (a barrier) and refilled with the step after next
// there: each step's loads have a step and a half of MFMAs to land in.
template <int EPI, int WTN>
__global__ __attribute__((amdgpu_flat_work_group_size(GW * 64, GW * 64), amdgpu_waves_per_eu(1, 1)))
void gemm256_kernel(GemmParams p) {
  constexpr int BN = 32 * WTN;     // tile columns
  constexpr int NBP = WTN / 2;     // block pairs of B per wave and step
  constexpr int NLD = 2 * (4 + NBP);  // load instructions per wave and step
  static_assert(WTN == 8 || WTN == 6, "tile widths of this kernel");
  __shared__ __attribute__((aligned(16))) bf16 sA[2][GBM2 * GBK];
  __shared__ __attribute__((aligned(16))) bf16 sB[2][BN * GBK];

  int mt, nt;
  xcd_remap(blockIdx.x, p.mtiles, p.ntiles, mt, nt);
  const int64_t m0 = (int64_t)mt * GBM2;
  const int n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int li = lane & 15, lg = lane >> 4;
  const int nk = p.K / GBK;

  // Direct-to-LDS loads (global_load_lds_dwordx4): lane l of one instruction
  // writes LDS bytes [16 l, 16 l + 16) of a 1 KB block, which is 8 rows of a
  // 256 x 64 tile in tile_off's layout; lane l takes row l / 8 at chunk
  // position l % 8, so it loads logical chunk (l % 8) ^ (l / 8) of that row.
  // M and N are multiples of 8 and K of 64 on this path, so a block of rows
  // lies wholly inside or wholly past the matrix; one past it loads the last
  // 8 rows instead, which are never stored.  The block's first row is
  // uniform (a scalar base address); the lane's byte offset within it is the
  // same for every block and step.  They are written as inline assembly so
  // that the compiler, which cannot tell a buffer being filled from one being
  // read, does not wait for them before every LDS read: the loop waits for
  // them itself.
  const int r8 = lane >> 3;
  const uint32_t loff = (uint32_t)(r8 * p.K + (((lane & 7) ^ r8) << 3)) * 2u;
  const uint32_t lds_a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16*)&sA[0][0];
  const uint32_t lds_b = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16*)&sB[0][0];
  // A wave fills 8 consecutive 1 KB blocks of the A tile and WTN of the B
  // tile.  The instruction's offset field moves both the LDS destination and
  // the global address, so one M0 value (the wave's span + 4 KB) serves all of
  // a tile's blocks with offsets -4096 .. 3072; each block's scalar base is
  // lowered by its offset.  (Rewriting M0 before every load measurably stalls
  // the issuing wave.)  dma(kt, buf, q) loads blocks 2q, 2q + 1 of A (q < 4)
  // or 2(q - 4), 2(q - 4) + 1 of B (4 <= q < 4 + NBP).
  auto dma = [&](int kt, int buf, int q) {
    const bool isb = q >= 4;
    const int i0 = (q & 3) * 2;
    const int blk0 = wave * (isb ? WTN : 8) + i0;
    const int64_t lim = isb ? (int64_t)p.N - 8 : p.M - 8;
    const int64_t r0 = min((isb ? (int64_t)n0 : m0) + blk0 * 8, lim);
    const int64_t r1 = min((isb ? (int64_t)n0 : m0) + blk0 * 8 + 8, lim);
    const bf16* src = isb ? p.b : p.a;
    const int off0 = i0 * 1024 - 4096;
    const char* g0 = reinterpret_cast<const char*>(src + r0 * p.K + kt * GBK) - off0;
    const char* g1 = reinterpret_cast<const char*>(src + r1 * p.K + kt * GBK) - (off0 + 1024);
    const uint32_t m0v = isb ? lds_b + (uint32_t)(buf * BN * GBK + wave * WTN * 512) * 2u + 4096u
                             : lds_a + (uint32_t)(buf * GBM2 * GBK + wave * 8 * 512) * 2u + 4096u;
    // one wait state between writing M0 and the first load
#define BCA_DMA2(O0, O1)                                                                        \
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:" #O0                          \
               "\n\tglobal_load_lds_dwordx4 %0, %2 offset:" #O1 ::"v"(loff), "s"(g0), "s"(g1), \
               "{m0}"(m0v)                                                                      \
               : "memory")
    switch (q & 3) {
      case 0: BCA_DMA2(-4096, -3072); break;
      case 1: BCA_DMA2(-2048, -1024); break;
      case 2: BCA_DMA2(0, 1024); break;
      default: BCA_DMA2(2048, 3072); break;
    }
#undef BCA_DMA2
  };

  f32x4 acc[WTN][WT];  // [n tile][m tile] of C^T
#pragma unroll
  for (int i = 0; i < WTN; ++i)
#pragma unroll
    for (int j = 0; j < WT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // operands of one 32-wide k slice: WTN tiles of B rows, 8 of A rows
  auto rd_b = [&](int buf, int ks, int t) {
    return ld_lds16(&sB[buf][0] + tile_off(wn * 16 * WTN + t * 16 + li, ks * 4 + lg));
  };
  auto rd_a = [&](int buf, int ks, int t) {
    return ld_lds16(&sA[buf][0] + tile_off(wm * 128 + t * 16 + li, ks * 4 + lg));
  };

#pragma unroll
  for (int q = 0; q < 4 + NBP; ++q) dma(0, 0, q);
#pragma unroll
  for (int q = 0; q < 4 + NBP; ++q) dma(min(1, nk - 1), 1, q);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NLD) : "memory");  // step 0 has landed
  __syncthreads();
  // Branches inside a step, where the accumulators are live, make the
  // register allocator shuffle them, so every step refills: the last two
  // reload the last step's tiles into a buffer no later step reads.
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    // first half: the first slice's operands, then its 64 MFMAs with the
    // second slice's reads between them (scheduling fences keep the order)
    bf16x8 b0[WTN], a0[WT], b1[WTN], a1[WT];
#pragma unroll
    for (int t = 0; t < WT; ++t) a0[t] = rd_a(buf, 0, t);
#pragma unroll
    for (int t = 0; t < WTN; ++t) b0[t] = rd_b(buf, 0, t);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < WTN; ++i) {
#pragma unroll
      for (int j = 0; j < WT; ++j) acc[i][j] = mfma16(b0[i], a0[j], acc[i][j]);
      a1[i] = rd_a(buf, 1, i);
      b1[i] = rd_b(buf, 1, i);
      if (i == WTN - 1) {
#pragma unroll
        for (int t = WTN; t < WT; ++t) a1[t] = rd_a(buf, 1, t);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // mid-step: once every wave's reads of this buffer have completed it
    // takes the step after next
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // second half: the second slice's MFMAs with the refill's loads spread
    // between them (a burst of loads would stall the wave's MFMA issue)
    const int kn = min(kt + 2, nk - 1);
#pragma unroll
    for (int i = 0; i < WTN; ++i) {
#pragma unroll
      for (int j = 0; j < WT; ++j) acc[i][j] = mfma16(b1[i], a1[j], acc[i][j]);
      dma(kn, buf, i);
      if (i == WTN - 1) {
#pragma unroll
        for (int q = WTN; q < 4 + NBP; ++q) dma(kn, buf, q);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // end of step: the next step's loads (issued before this step's refill)
    // have landed in every wave
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NLD) : "memory");
    __syncthreads();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the surplus reloads land before the workgroup ends

  // The results leave through LDS, 16 rows at a time per wave, so that
  // each lane stores (and, with a residual, loads) 16 contiguous bytes
  // and consecutive lanes continue along a row: the accumulator layout
  // would give 8-byte pieces 16 rows apart.  Every wave's direct-to-LDS
  // loads have landed before the buffers are reused.
  __syncthreads();
  constexpr int CW = 16 * WTN;  // the wave's columns
  constexpr int SP = CW + 4;    // padded row stride (floats): rows 4 banks apart
  constexpr int PER = CW / 8;   // 8-column pieces per row
  static_assert((16 * PER) % 64 == 0 && 4 * 16 * SP * 4 <= (int)sizeof(sA), "epilogue staging");
  float* slab = reinterpret_cast<float*>(&sA[0][0]) + wave * 16 * SP;
  const int64_t mw = m0 + wm * 128;
  const int nw = n0 + wn * CW;
  constexpr int IT = 16 * PER / 64;  // pieces per lane and 16-row round
  // the residual pieces of every round, issued together (one latency)
  constexpr bool PRE = EPI == 1;
  bf16x8 res[PRE ? WT : 1][PRE ? IT : 1];
  if constexpr (PRE) {
#pragma unroll
    for (int j = 0; j < WT; ++j)
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int k = lane + 64 * it;
        const int r = k / PER, c = (k - (k / PER) * PER) * 8;
        const int64_t m = min(mw + j * 16 + r, p.M - 1);
        res[j][it] = p.residual ? ld_global16(p.residual + m * p.N + min(nw + c, p.N - 8)) : zero8();
      }
  }
#pragma unroll
  for (int j = 0; j < WT; ++j) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < WTN; ++i)
      *reinterpret_cast<f32x4*>(slab + li * SP + i * 16 + lg * 4) = acc[i][j];
#pragma unroll
    for (int it = 0; it < 16 * PER / 64; ++it) {
      const int k = lane + 64 * it;
      const int r = k / PER, c = (k - (k / PER) * PER) * 8;
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(slab + r * SP + c);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(slab + r * SP + c + 4);
      if constexpr (PRE)
        store8r(p, mw + j * 16 + r, nw + c, v0, v1, res[j][it]);
      else
        store8<EPI>(p, mw + j * 16 + r, nw + c, v0, v1);
    }
  }
}

// One wave per row: rstd = 1/sqrt(mean(x^2) + eps) in fp32.  Rows are
// d_model elements, d_model % 8 == 0.
__global__ __launch_bounds__(256) void rstd_rows_kernel(const bf16* x, float eps, int64_t M, int dm,
                                                        float* rstd_out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const bf16* xr = x + row * dm;
  const int nch = dm >> 3;
  float ss = 0.f;
  // four 16-byte pieces per lane in flight at once (rows of up to 2048)
  int c = lane;
  for (; c + 192 < nch; c += 256) {
    bf16x8 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ld_global16(xr + (c + 64 * i) * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) ss = sumsq8(v[i], ss);
  }
  bf16x8 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = c + 64 * i < nch ? ld_global16(xr + (c + 64 * i) * 8) : zero8();
#pragma unroll
  for (int i = 0; i < 4; ++i) ss = sumsq8(v[i], ss);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if (lane == 0) rstd_out[row] = 1.0f / sqrtf(ss / (float)dm + eps);
}

// The RMS norm's gain folded into the QKV weights: wf[n][c] = bf16(w[n][c] *
// gain[c]), one thread per 8 elements (K % 8 == 0).
__global__ __launch_bounds__(256) void fold_gain_kernel(const bf16* w, const float* gain, int64_t count,
                                                        int K, bf16* wf) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  const int c = (int)((i * 8) % K);
  const bf16x8 v = ld_global16(w + i * 8);
  const f32x4 g0 = *reinterpret_cast<const f32x4*>(gain + c);
  const f32x4 g1 = *reinterpret_cast<const f32x4*>(gain + c + 4);
  f32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = (float)v[e] * g0[e];
    b[e] = (float)v[4 + e] * g1[e];
  }
  st_global16(wf + i * 8, pack8(a, b));
}

hipError_t launch_gemm(GemmParams& p, int epi, hipStream_t stream) {
  // the lane offset of gemm256_kernel's loads is a 32-bit byte count < 16 K
  const bool big = p.M >= 8 && p.N >= 8 && p.M % 8 == 0 && p.N % 8 == 0 && p.K % GBK == 0 &&
                   p.K <= (1 << 24);
  const bool n192 = big && p.N % 192 == 0 && p.N % 256 != 0;
  const int bm = big ? GBM2 : GBM, bn = n192 ? 192 : big ? GBN2 : GBN;
  p.mtiles = (int)((p.M + bm - 1) / bm);
  p.ntiles = (p.N + bn - 1) / bn;
  const int64_t grid = (int64_t)p.mtiles * p.ntiles;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidValue;
  auto k = n192  ? (epi == 0 ? gemm256_kernel<0, 6> : gemm256_kernel<1, 6>)
           : big ? (epi == 0 ? gemm256_kernel<0, 8> : gemm256_kernel<1, 8>)
                 : (epi == 0 ? gemm_nt_kernel<0> : gemm_nt_kernel<1>);
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(GW * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm_qkv(const ProjDims& d, const void* x, const float* gain, float eps,
                              const void* w, void* q, void* k, void* v, float* rstd,
                              void* workspace, hipStream_t stream) {
  GemmParams p{};
  p.a = static_cast<const bf16*>(x);
  p.M = d.M;
  p.N = (d.Hq + 2 * d.Hkv) * d.D;
  p.K = d.d_model;
  p.out0 = static_cast<bf16*>(q);
  p.out1 = static_cast<bf16*>(k);
  p.out2 = static_cast<bf16*>(v);
  p.nq = d.Hq * d.D;
  p.nkv = d.Hkv * d.D;
  // workspace: the gain-folded weights, then room for rstd
  bf16* wf = static_cast<bf16*>(workspace);
  float* rs = rstd ? rstd : reinterpret_cast<float*>(static_cast<char*>(workspace) + qkv_weight_bytes(d));
  const int64_t n8 = (int64_t)p.N * p.K / 8;
  hipLaunchKernelGGL(fold_gain_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const bf16*>(w), gain, n8, p.K, wf);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  p.b = wf;
  const int64_t blocks = (d.M + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rstd_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p.a, eps, d.M,
                     d.d_model, rs);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  p.rstd_in = rs;
  return launch_gemm(p, 0, stream);
}

hipError_t launch_out_proj(const ProjDims& d, const void* o, const void* w, const void* residual,
                           void* y, hipStream_t stream) {
  GemmParams p{};
  p.a = static_cast<const bf16*>(o);
  p.b = static_cast<const bf16*>(w);
  p.M = d.M;
  p.N = d.d_model;
  p.K = d.Hq * d.D;
  p.out0 = static_cast<bf16*>(y);
  p.residual = static_cast<const bf16*>(residual);
  return launch_gemm(p, 1, stream);
}

}  // namespace bca
