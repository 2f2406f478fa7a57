// Flash-style forward of space and time attention, bf16 in/out, head_dim 64,
// for gfx950 (MI355X).
//
// Open Dreamer articles (pro.edgex.exchange, fr-FR edition): section
// "Architecture" (space layers inside one timestep block, causal time layers
// across frames, world tokens cannot read the agent token) and section
// "Configuration d'entraînement" (GQA 30 query heads over 3 KV heads, 192-step
// sliding window for time attention).  Mixed precision follows the section
// "Ingénierie de la stabilité": bf16 attention inputs, fp32 statistics.
//
// Work decomposition.  One attention problem is a (unit, KV head g) pair: a
// unit is a block (space: positions = the N tokens of one frame) or a token
// slot (time: positions = the T frames).  Its G = Hq/Hkv query heads are
// folded into rows r = position * G + head-in-group, so that the K/V of the
// group, staged once in LDS, serve all G heads.  A workgroup owns a
// contiguous row range of one problem; each of its 8 waves takes 32-row
// chunks and sweeps the visible keys in 32-key steps.
//
// Per step and wave: S^T (keys x queries) = K Q^T on MFMA with K from LDS and
// Q^T from registers, so every lane holds one query column and the row
// statistics need only a 4-lane reduction; online softmax in the log2 domain
// with a lazy rescale (a row's running reference max is moved only when one
// of its new scores exceeds it by more than 2^8, which keeps exp2 arguments
// <= 8; rows never rescale because of other rows' scores; after a chunk's
// first step the exps are formed first and that exact test runs only when
// some lane's 8 exps of a row sum to more than 2^8);
// O^T += V^T P^T on MFMA, V kept row-major in LDS (laid out as K, one 16-byte
// write per piece when staged) and its V^T operand formed by transposing LDS
// reads.  Fully masked key steps are never
// visited (causal and window ranges), and per-element masks are applied only
// on steps that straddle a mask edge.
#include <type_traits>

#include "bca_device.h"
#include "bca_kernels.h"

namespace bca {

namespace {

constexpr int KMAX = 320;   // keys resident in LDS per pass
constexpr int FW = 8;       // waves per workgroup
constexpr int QCH = 32;     // query rows per wave and chunk
// decode: small workgroups with a small key block, so that several
// problems (each one computing wave) share a CU and their staging overlaps
constexpr int DEC_FW = 4;
constexpr int DEC_KMAX = 96;
template <int OP> constexpr int waves_of() { return OP == OP_DECODE ? DEC_FW : FW; }
template <int OP> constexpr int keys_of() { return OP == OP_DECODE ? DEC_KMAX : KMAX; }
constexpr int NQT = QCH / 16;
constexpr float kRescaleThreshold = 8.0f;  // log2 units

struct FwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  int T, N, Hq, Hkv, G, L, units, rows;
  int window, agent_begin, agent_count;
  float scale_log2, inv_g;
  float inv_scale_log2;  // 1 / scale_log2
  int splits, rows_per_split;
  // decode: K/V hold Tk frames per slot; kernel key position x is absolute
  // frame kfirst + x at frame (kfirst + x) % Tk; kernel query position y sits
  // at key position y + qoff
  int Tk, kfirst, qoff;
  int poison;  // debug: NaN-fill LDS before staging
};

// sK, sV: [KMAX][64], 16-byte pieces xor-swizzled by row
__device__ __forceinline__ int k_off(int row, int chunk) {
  return row * 64 + ((chunk ^ (row & 7)) << 3);
}

// 8 waves of 32 query rows; two workgroups (80 KB of LDS each) share a CU,
// so each SIMD interleaves four waves.  OP_DECODE runs the time op's code
// with the query positions shifted by qoff and the key frames read from a
// ring (rollout over a KV cache); its chunks are 16 rows (a problem has G
// rows per new frame); since its staging, not its few steps, dominates, a
// decode workgroup is 4 waves with a 96-key block (24 KB of LDS), so five
// problems share a CU, and each thread issues all its loads of a block
// before its LDS stores.
template <int OP>
__global__ __attribute__((amdgpu_flat_work_group_size(waves_of<OP>() * 64, waves_of<OP>() * 64),
                          amdgpu_waves_per_eu(4, 4)))
void attn_fwd_kernel(FwdParams p) {
  constexpr int FW = waves_of<OP>();
  constexpr int KMAX = keys_of<OP>();
  // rows per chunk: a decode problem has only G rows per new frame
  constexpr int NQ = OP == OP_DECODE ? 1 : NQT;
  constexpr int QC = 16 * NQ;
  __shared__ __attribute__((aligned(16))) bf16 sK[KMAX * 64];
  __shared__ __attribute__((aligned(16))) bf16 sV[KMAX * 64];
  constexpr int NT = FW * 64;
  if (p.poison) {
    poison_lds(sK, sizeof(sK), threadIdx.x, NT);
    poison_lds(sV, sizeof(sV), threadIdx.x, NT);
    __syncthreads();
  }

  int ug, split;
  if constexpr (OP == OP_TIME) {
    // causal rows: later row splits see more keys, so they are dispatched
    // first and the lighter early splits fill the grid's last round
    const int P = p.units * p.Hkv;
    const int sidx = blockIdx.x / P;
    split = p.splits - 1 - sidx;
    ug = blockIdx.x - sidx * P;
  } else {
    xcd_remap(blockIdx.x, p.units * p.Hkv, p.splits, ug, split);
  }
  const int u = ug / p.Hkv, g = ug - (ug / p.Hkv) * p.Hkv;
  constexpr int MOP = OP == OP_DECODE ? OP_TIME : OP;  // mask and layout kind
  const int qsh = OP == OP_DECODE ? p.qoff : 0;        // query -> key position
  const UnitGeom gq = unit_geom(MOP, u, p.T, p.N, p.Hq, 64);
  const UnitGeom gk = unit_geom(MOP, u, p.Tk, p.N, p.Hkv, 64);
  const UnitGeom gl = unit_geom(MOP, u, p.T, p.N, p.Hq, 1);
  const MaskDesc md{MOP, p.L, p.window, p.agent_begin, p.agent_count};
  const unsigned weff = (unsigned)(p.window > 0 ? p.window : p.L);
  auto kframe = [&](int x) { return OP == OP_DECODE ? (p.kfirst + x) % p.Tk : x; };
  const bf16* kbase = p.k + gk.base + g * 64;
  const bf16* vbase = p.v + gk.base + g * 64;
  const bf16* qbase = p.q + gq.base + (int64_t)g * p.G * 64;
  bf16* obase = p.o + gq.base + (int64_t)g * p.G * 64;
  float* lbase = p.lse + gl.base + g * p.G;

  const int row0 = split * p.rows_per_split;
  const int row1 = min(p.rows, row0 + p.rows_per_split);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int li = lane & 15, lg = lane >> 4;
  const int nch = (row1 - row0 + QC - 1) / QC;
  const int passes = (nch + FW - 1) / FW;
  const int G = p.G;
  // keys [wklo, wkhi) are all that any row of this workgroup sees (32-key
  // aligned start); they pass through LDS in blocks of up to KMAX keys
  int wklo, wkhi;
  key_range(md, row0 / G + qsh, (row1 - 1) / G + qsh, wklo, wkhi);
  wklo &= ~31;
  const int nkb = (wkhi - wklo + KMAX - 1) / KMAX;

  // this lane's query column in each 16-column tile of a chunk; padding
  // columns read a real (clamped) row and are never stored.  The next
  // chunk's Q is loaded before this chunk's O is stored, so that the first
  // products of the next chunk do not wait behind the stores.
  bf16x8 qreg[NQ][2];
  auto load_q = [&](int pass) {
    const int r0n = row0 + (pass * FW + wave) * QC;
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt) {
      const int rr = min(r0n + qt * 16 + li, row1 - 1);
      const int pos = row_pos(rr, p.inv_g);
      const bf16* src = qbase + pos * gq.pos_stride + (rr - pos * G) * 64 + lg * 8;
      qreg[qt][0] = ld_global16(src);
      qreg[qt][1] = ld_global16(src + 32);
    }
  };
  if (wave < nch) load_q(0);
  for (int pass = 0; pass < passes; ++pass) {
    const int ch = pass * FW + wave;
    const bool active = ch < nch;
    const int r0 = row0 + ch * QC;

    int qpos[NQ], hh[NQ];
    bool qvalid[NQ];
    f32x4 acc[NQ][4];
    float m[NQ], l[NQ];
    // per row, kept in step with m: -m (0 while m = -inf) for the exp
    // argument, and the raw-score threshold (m + 2^8 in log2 units, divided
    // by the scale) above which the row may need a new reference
    float negm[NQ], thr[NQ];
    // and the bound on the sum of a lane's 8 exps of the row in one step
    // above which the exact test runs: 2^8, or -1 (always) while the row
    // has no reference yet
    float lim[NQ];
    bool fresh = true;  // no step of the chunk visited yet
    int qlo = 0, qhi = 0;
    if (active) {
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt) {
        const int r = r0 + qt * 16 + li;
        qvalid[qt] = r < row1;
        const int rr = min(r, row1 - 1);
        qpos[qt] = row_pos(rr, p.inv_g);
        hh[qt] = rr - qpos[qt] * G;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[qt] = -INFINITY;
        negm[qt] = 0.f;
        thr[qt] = -INFINITY;
        lim[qt] = -1.f;
        l[qt] = 0.f;
      }
      qlo = r0 / G + qsh;
      qhi = (min(r0 + QC, row1) - 1) / G + qsh;
    }

    for (int kb = 0; kb < nkb; ++kb) {
      const int key0 = wklo + kb * KMAX;
      const int kn = min(KMAX, wkhi - key0);
      if (nkb > 1 || pass == 0) {
        if (nkb > 1) __syncthreads();
        const int lp = (kn + 31) & ~31;
        if constexpr (OP == OP_DECODE) {
          constexpr int PER = KMAX * 8 / NT;
          static_assert(PER * NT == KMAX * 8, "a block is a whole number of rounds");
          bf16x8 kq[PER], vq[PER];
#pragma unroll
          for (int i = 0; i < PER; ++i) {
            const int idx = tid + i * NT, r = idx >> 3, c = idx & 7;
            kq[i] = zero8();
            vq[i] = zero8();
            if (r < kn) {
              kq[i] = ld_global16(kbase + (int64_t)kframe(key0 + r) * gk.pos_stride + c * 8);
              vq[i] = ld_global16(vbase + (int64_t)kframe(key0 + r) * gk.pos_stride + c * 8);
            }
          }
#pragma unroll
          for (int i = 0; i < PER; ++i) {
            const int idx = tid + i * NT, r = idx >> 3, c = idx & 7;
            if (r < lp) {
              st_lds16(sK + k_off(r, c), kq[i]);
              st_lds16(sV + k_off(r, c), vq[i]);
            }
          }
        } else {
          for (int idx = tid; idx < lp * 8; idx += NT) {
            const int r = idx >> 3, c = idx & 7;
            bf16x8 kv = zero8(), vv = zero8();
            if (r < kn) {
              kv = ld_global16(kbase + (int64_t)kframe(key0 + r) * gk.pos_stride + c * 8);
              vv = ld_global16(vbase + (int64_t)kframe(key0 + r) * gk.pos_stride + c * 8);
            }
            st_lds16(sK + k_off(r, c), kv);
            st_lds16(sV + k_off(r, c), vv);
          }
        }
        __syncthreads();
      }
      if (!active) continue;

      int klo, khi;
      key_range(md, qlo, qhi, klo, khi);
      klo = max(klo, key0);
      khi = min(khi, key0 + kn);
      if (klo >= khi) continue;
      const int st0 = (klo - key0) >> 5, st1 = (khi - key0 + 31) >> 5;
      // one 32-key step; FIRST: the chunk's first visited step, which sets
      // the rows' references before forming any exp
      auto step = [&](int st, auto first_c) {
        constexpr bool FIRST = decltype(first_c)::value;
        const int kabs = key0 + st * 32;
        // S^T tiles: rows = 16 keys (two halves of the step), columns = queries
        f32x4 sc[NQ][2];
        auto scores = [&](int kst) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int kr = kst + h * 16 + li;
            const bf16x8 k0 = ld_lds16(sK + k_off(kr, lg));
            const bf16x8 k1 = ld_lds16(sK + k_off(kr, 4 + lg));
#pragma unroll
            for (int qt = 0; qt < NQ; ++qt) {
              f32x4 z = {0.f, 0.f, 0.f, 0.f};
              z = mfma16(k0, qreg[qt][0], z);
              sc[qt][h] = mfma16(k1, qreg[qt][1], z);
            }
          }
          // hipcc leaves as few as 7 wait states between these MFMAs and the
          // first VALU read of sc along the branch paths below (8 are needed);
          // a fixed pad covers every path
          __builtin_amdgcn_sched_barrier(0);
          asm volatile("s_nop 7" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
          if (!tile_all_visible(md, qlo, qhi, kabs, kabs + 32)) {
            // a select, not a conditional store: hipcc dropped conditional
            // element stores into this array of vectors
#pragma unroll
            for (int qt = 0; qt < NQ; ++qt) {
              // time: the query sits at a real position (< L), so a key is
              // visible iff 0 <= query - key < window (the whole sequence when
              // there is none): one unsigned compare, and keys past the end
              // fail it too
              const int dq0 = qpos[qt] + qsh - kabs - lg * 4;
#pragma unroll
              for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  bool vis;
                  if constexpr (MOP == OP_TIME)
                    vis = (unsigned)(dq0 - h * 16 - j) < weff;
                  else
                    vis = visible_op<MOP>(md, qpos[qt] + qsh, kabs + h * 16 + lg * 4 + j);
                  const float cur = sc[qt][h][j];
                  sc[qt][h][j] = vis ? cur : -INFINITY;
                }
            }
          }
        };
        scores(st * 32);
        // The exps are formed against the current references first (except
        // on the chunk's first step); a lane whose 8 exps of a row sum to at
        // most 2^8 has none above 2^8, so none of its scores could move the
        // reference, and only when some lane of the wave exceeds that bound
        // does the wave form the scores again, run the exact test below and
        // form the exps anew
        f32x4 e0[NQ], e1[NQ];
        float ls[NQ];  // sum of the lane's 8 exps of the row
        auto form_exps = [&]() {
#pragma unroll
          for (int qt = 0; qt < NQ; ++qt) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              e0[qt][j] = fast_exp2(__builtin_fmaf(sc[qt][0][j], p.scale_log2, negm[qt]));
              e1[qt][j] = fast_exp2(__builtin_fmaf(sc[qt][1][j], p.scale_log2, negm[qt]));
            }
            ls[qt] = ((e0[qt][0] + e0[qt][1]) + (e0[qt][2] + e0[qt][3])) +
                     ((e1[qt][0] + e1[qt][1]) + (e1[qt][2] + e1[qt][3]));
          }
        };
        bool check = FIRST;
        if constexpr (!FIRST) {
          form_exps();
          bool big = false;
#pragma unroll
          for (int qt = 0; qt < NQ; ++qt) big |= ls[qt] > lim[qt];
          check = __builtin_amdgcn_ballot_w64(big) != 0;
          if (check) {
            // the scores again rather than held through the exps (registers);
            // the opaque offset keeps the compiler from reusing the first ones
            int kst = st * 32;
            asm volatile("" : "+s"(kst));
            scores(kst);
          }
        }
        if (check) {
          // online softmax with a lazy reference max (log2 domain): a row's
          // reference moves only when one of its scores exceeds it by more
          // than 2^8, and only that row is rescaled (the others multiply by
          // exactly 1), so every row depends on its own scores alone
          // each lane first tests its own 8 scores of the row; the 4-lane
          // row maximum is formed only when some lane of the wave is over
          float lmx[NQ];  // raw (unscaled) maximum of the lane's 8 scores of the row
          bool over = false;
#pragma unroll
          for (int qt = 0; qt < NQ; ++qt) {
            const float a = fmaxf(fmaxf(sc[qt][0][0], sc[qt][0][1]), fmaxf(sc[qt][0][2], sc[qt][0][3]));
            const float b = fmaxf(fmaxf(sc[qt][1][0], sc[qt][1][1]), fmaxf(sc[qt][1][2], sc[qt][1][3]));
            lmx[qt] = fmaxf(a, b);
            over |= lmx[qt] > thr[qt];
          }
          if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
            for (int qt = 0; qt < NQ; ++qt) {
              // the scale is positive, so scaling commutes with the maximum
              const float mx = group4_max(lmx[qt]) * p.scale_log2;
              const bool grow = mx > m[qt] + kRescaleThreshold;
              const float mn = grow ? mx : m[qt];
              const float alpha = grow ? fast_exp2(m[qt] - mn) : 1.f;
              l[qt] *= alpha;
#pragma unroll
              for (int dt = 0; dt < 4; ++dt) acc[qt][dt] *= alpha;
              m[qt] = mn;
              negm[qt] = (mn == -INFINITY) ? 0.f : -mn;
              // (the bound only decides when the test above runs; an ulp
              // either way can change whether a score right at the threshold
              // moves the reference, which the results do not depend on
              // beyond rounding)
              thr[qt] = (mn + kRescaleThreshold) * p.inv_scale_log2;
            lim[qt] = (mn == -INFINITY) ? -1.f : 256.f;
            }
          }
          form_exps();
        }
        bf16x8 pb[NQ];
#pragma unroll
        for (int qt = 0; qt < NQ; ++qt) {
          l[qt] += ls[qt];
          pb[qt] = pack8(e0[qt], e1[qt]);
        }
        // O^T += V^T P^T.  Tile dt's operand row r is head dim 8 (r >> 2) +
        // 4 (dt & 1) + 32 (dt >> 1) + (r & 3), so that its output rows 4 lg
        // .. 4 lg + 3 are dims 8 lg + 4 (dt & 1) + 32 (dt >> 1) .. +3: each
        // lane ends with dims 8 lg .. +7 and 32 + 8 lg .. +7 of its query
        // row, and each of its two 16-byte stores joins the other lanes of
        // the row into 64 contiguous bytes.  Lane (li, lg) receives dim 8
        // (li >> 2) + 4 (dt & 1) + 32 (dt >> 1) + (li & 3) of keys 4 lg .. +3
        // and 16 + 4 lg .. +3 of the step, the keys its P^T operand holds:
        // the lanes with li & 3 == b address the four dims from 8 b + ....
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int kr = st * 32 + 4 * lg + (li >> 2), dcol = 8 * (li & 3) + 4 * (dt & 1) + 32 * (dt >> 1);
          const bf16x8 vt = join8(ld_lds_tr4(sV + k_off(kr, dcol >> 3) + (dcol & 7)),
                                  ld_lds_tr4(sV + k_off(kr + 16, dcol >> 3) + (dcol & 7)));
#pragma unroll
          for (int qt = 0; qt < NQ; ++qt) acc[qt][dt] = mfma16(vt, pb[qt], acc[qt][dt]);
        }
      };
      int st = st0;
      if (fresh) {
        fresh = false;
        step(st++, std::true_type{});
      }
      for (; st < st1; ++st) step(st, std::false_type{});
    }

    if (active) {
      if (ch + FW < nch) load_q(pass + 1);
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt) {
        const float lt = group4_sum(l[qt]);
        if (!qvalid[qt]) continue;
        const float inv = __builtin_amdgcn_rcpf(lt);  // (O is rounded to bf16)
        // dims 8 lg .. +7 and 32 + 8 lg .. +7 of the row
        bf16* dst = obase + qpos[qt] * gq.pos_stride + hh[qt] * 64 + lg * 8;
        st_global16(dst, pack8(acc[qt][0] * inv, acc[qt][1] * inv));
        st_global16(dst + 32, pack8(acc[qt][2] * inv, acc[qt][3] * inv));
        if (lg == 0) lbase[qpos[qt] * gl.pos_stride + hh[qt]] = (m[qt] + __log2f(lt)) * kLn2;
      }
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnDims& d, const void* q, const void* k, const void* v,
                                void* o, float* lse, hipStream_t stream) {
  FwdParams p;
  p.q = static_cast<const bf16*>(q);
  p.k = static_cast<const bf16*>(k);
  p.v = static_cast<const bf16*>(v);
  p.o = static_cast<bf16*>(o);
  p.lse = lse;
  p.T = d.T;
  p.N = d.N;
  p.Hq = d.Hq;
  p.Hkv = d.Hkv;
  p.G = d.Hq / d.Hkv;
  p.L = d.op == OP_SPACE ? d.N : d.T;
  p.units = d.op == OP_SPACE ? d.B * d.T : d.B * d.N;
  p.rows = p.L * p.G;
  p.Tk = d.T;
  p.kfirst = 0;
  p.qoff = 0;
  if (d.op == OP_DECODE) {
    int first, last;
    decode_key_range(d, first, last);
    p.L = last - first + 1;
    p.rows = d.T * p.G;
    p.Tk = d.kv_frames;
    p.kfirst = first;
    p.qoff = d.q_frame0 - first;
  }
  p.window = d.window;
  p.agent_begin = d.agent_begin;
  p.agent_count = d.agent_count;
  p.scale_log2 = d.scale * kLog2e;
  p.inv_scale_log2 = 1.0f / p.scale_log2;
  p.inv_g = 1.0f / (float)p.G;
  p.poison = d.poison;
  if (p.G > 256 || (long)p.rows >= (1L << 21)) return hipErrorInvalidValue;
  // Split each problem's rows over several workgroups so that the grid
  // covers the 256 CUs (two workgroups each) about three times over.
  const long problems = (long)p.units * p.Hkv;
  const int qch = d.op == OP_DECODE ? 16 : QCH;  // rows per chunk (as in the kernel)
  const int FW = d.op == OP_DECODE ? DEC_FW : bca::FW;  // waves per workgroup
  const int chunks = (p.rows + qch - 1) / qch;
  int splits = (int)((3 * 512 + problems - 1) / problems);
  // A grid too small to fill the chip that way (one block's space attention
  // during a rollout) is split down to 2 chunks per workgroup: more of the
  // chip then stages K/V and computes at once (1 chunk restages too much).
  splits = max(1, min(splits, (chunks + 1) / 2));
  int per = (chunks + splits - 1) / splits;
  if (per >= FW) per = ((per + FW - 1) / FW) * FW;  // whole passes of FW chunks
  // Windowed time attention over many frames: fewer rows per workgroup, so
  // that the keys a workgroup sees fit one LDS block (otherwise every pass
  // restages all its blocks).
  if (d.op == OP_TIME && p.window > 0)
    while (per > FW && time_wg_key_span(p.L, p.G, p.window, (long)per * qch) > KMAX) per -= FW;
  p.rows_per_split = per * qch;
  p.splits = (p.rows + p.rows_per_split - 1) / p.rows_per_split;
  const long grid = problems * p.splits;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidValue;
  if (d.op == OP_SPACE)
    hipLaunchKernelGGL(attn_fwd_kernel<OP_SPACE>, dim3((unsigned)grid), dim3(FW * 64), 0, stream, p);
  else if (d.op == OP_TIME)
    hipLaunchKernelGGL(attn_fwd_kernel<OP_TIME>, dim3((unsigned)grid), dim3(FW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<OP_DECODE>, dim3((unsigned)grid), dim3(DEC_FW * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace bca
