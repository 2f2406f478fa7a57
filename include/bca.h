/*
 * bca.h -- block-causal attention for AMD MI355X (gfx950): C ABI.
 *
 * The operations are the two attention kinds of the block-causal transformer
 * backbone shared by the Open Dreamer tokenizer and dynamics model (Open
 * Dreamer articles, pro.edgex.exchange fr-FR edition):
 *
 *  - space attention: section "Architecture" -- space layers move
 *    information among the tokens of one timestep block, and world-model
 *    tokens cannot read the agent token; section "Configuration
 *    d'entraînement" -- 30 query heads over 3 KV heads (grouped-query
 *    attention) at d_model 1920, i.e. head_dim 64.
 *  - time attention: section "Architecture" -- causal time layers move
 *    information across frames; section "Configuration d'entraînement" --
 *    a 192-step sliding window.
 *
 * Definition (softmax scale s, G = Hq / Hkv, query head h reads KV head
 * h / G).  A "unit" is one (b, t) block for space attention and one (b, n)
 * token slot for time attention; positions inside a unit are tokens
 * (space) or frames (time).  For query position i of head h:
 *     z_ij = s * <q_i,h , k_j,h/G>  for j in vis(i)
 *     O_i,h = sum_j softmax_j(z_i.) v_j,h/G,  LSE_i,h = ln sum_j exp(z_ij)
 * with
 *     space: vis(i) = { j : not agent(j) or agent(i) },
 *            agent(j) <=> agent_begin <= j < agent_begin + agent_count;
 *     time:  vis(t) = { t' : t' <= t and (window == 0 or t - t' <= window-1) }
 *            (the window counts the current frame).
 * The backward returns the gradients of sum(O * dO) with respect to q, k, v
 * (dK and dV of a KV head summed over the G query heads of its group).
 *
 * Layout (all row-major, contiguous):
 *     q, o, dout, dq : (B, T, N, Hq,  D)   dtype
 *     k, v, dk, dv   : (B, T, N, Hkv, D)   dtype
 *     lse            : (B, T, N, Hq)       float32, natural log
 * dtype is bf16 (BCA_BF16) or fp32 (BCA_F32); bf16 results are rounded to
 * nearest even from fp32 accumulators.  Supported head_dim: 32 and 64.
 *
 * Pointers are device pointers (HIP device memory of the current device),
 * 16-byte aligned.  The caller owns every buffer and keeps it alive until the
 * work queued on `stream` has finished.  Outputs are overwritten, never
 * accumulated, and must not alias inputs.  The library allocates no device
 * memory and keeps no state between calls; calls are thread-safe.
 *
 * Errors: every argument is validated on the host before anything is
 * launched; on failure nothing is written and a status is returned:
 *     BCA_ERR_INVALID_ARG  null pointer, non-positive size, Hq % Hkv != 0,
 *                          misaligned pointer, window < 0, agent range not
 *                          inside [0, N], workspace too small, sizes beyond
 *                          the 32-bit grid / 64-bit offset limits;
 *     BCA_ERR_UNSUPPORTED  head_dim not 32 or 64, unknown dtype, causal or
 *                          window set on the space op, causal == 0 on the
 *                          time op, more than 256 query heads per KV head
 *                          (G = Hq / Hkv), or 2^21 or more rows per problem
 *                          (attended length x G: N x G for space, T x G for
 *                          time, frames read x G for decode);
 *     BCA_ERR_HIP          the HIP runtime reported a launch error (any
 *                          error already pending in the calling thread's HIP
 *                          state is cleared first, so it is not reported).
 * bca_last_error() returns a human-readable detail of the calling thread's
 * last failure.  Work is asynchronous on `stream` (a hipStream_t; NULL = the
 * default stream); faults inside a kernel surface at the caller's next
 * synchronization.  No exception, abort or print crosses this interface.
 *
 * Non-finite inputs: inputs are expected to be finite.  A NaN or infinity in
 * the data of one problem -- one (unit, KV head) pair: the q, o, dout, lse
 * rows of its G query heads and the k, v rows of its KV head -- may leave
 * that problem's outputs NaN, infinite or meaningless; the outputs of every
 * other problem are exactly those of a run without it, and nothing faults.
 *
 * Debug switches (environment variables, read at every call; not for use
 * under stream capture):
 *     BCA_SYNC=1              every call synchronizes its stream after the
 *                             launch and returns BCA_ERR_HIP if a kernel
 *                             faulted;
 *     BCA_DEBUG_LDS_POISON=1  the attention kernels fill their LDS with NaN
 *                             bit patterns before staging, so that a read of
 *                             LDS no thread wrote shows up in the results.
 */
#ifndef BCA_H
#define BCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BCA_ABI_VERSION 4

typedef enum {
  BCA_OK = 0,
  BCA_ERR_INVALID_ARG = 1,
  BCA_ERR_UNSUPPORTED = 2,
  BCA_ERR_HIP = 3
} bca_status;

typedef enum { BCA_BF16 = 0, BCA_F32 = 1 } bca_dtype;

typedef enum { BCA_OP_SPACE = 0, BCA_OP_TIME = 1 } bca_op;

/* Tensor sizes: batch, frames, tokens per frame, query heads, KV heads,
 * head_dim, and the storage dtype (bca_dtype). */
typedef struct {
  int32_t B, T, N, Hq, Hkv, D;
  int32_t dtype;
} bca_shape;

/* Mask descriptor.
 *   causal        time op: must be 1 (t' <= t).  space op: must be 0.
 *   window        time op: > 0 -> key frame t' visible iff t - t' <= window-1;
 *                 0 -> unbounded causal.  space op: must be 0.
 *   agent_begin,  space op: slots [agent_begin, agent_begin + agent_count)
 *   agent_count   of every block are agent tokens, unreadable by the other
 *                 (world) tokens; agent tokens read every slot.  count 0 = no
 *                 isolation.  time op: validated, no effect (query and key
 *                 always share a slot).
 *   softmax_scale <= 0 -> 1/sqrt(D). */
typedef struct {
  int32_t causal;
  int32_t window;
  int32_t agent_begin;
  int32_t agent_count;
  float softmax_scale;
} bca_mask;

/* Space attention forward: writes o and lse.  Every query sees at least
 * itself, so no row is empty. */
int space_attn_fwd(const bca_shape* shape, const bca_mask* mask, const void* q,
                   const void* k, const void* v, void* o, float* lse, void* stream);

/* Space attention backward.  Inputs: q, k, v, the forward's o and lse, and
 * dout = dL/dO.  Outputs: dq, dk, dv.  workspace: device scratch of at least
 * bca_bwd_workspace_bytes(BCA_OP_SPACE, shape) bytes (may be NULL when that
 * is 0); its contents on entry do not matter. */
int space_attn_bwd(const bca_shape* shape, const bca_mask* mask, const void* q,
                   const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Causal sliding-window time attention forward (per token slot). */
int time_attn_fwd(const bca_shape* shape, const bca_mask* mask, const void* q,
                  const void* k, const void* v, void* o, float* lse, void* stream);

/* Causal sliding-window time attention backward; arguments as space_attn_bwd. */
int time_attn_bwd(const bca_shape* shape, const bca_mask* mask, const void* q,
                  const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Rollout decode of time attention (forward only).  Open Dreamer articles
 * (pro.edgex.exchange, fr-FR edition), section "Artefacts publiés": the
 * pipeline generates rollouts and the demo streams the generated world frame
 * by frame; section "Architecture": time layers are causal across frames.
 * Generating new frames runs the time op restricted to their query rows, with
 * the keys and values of earlier frames read from a cache.
 *
 *   shape->T       number of new (query) frames per slot, absolute frame
 *                  indices q_frame0 .. q_frame0 + T - 1;
 *   q, o           (B, T, N, Hq, D), lse (B, T, N, Hq) float32;
 *   k_cache,       (B, cache_frames, N, Hkv, D): a ring holding absolute frame
 *   v_cache        f at frame position f % cache_frames.  The caller writes the
 *                  new frames' K and V into the ring before the call;
 *   mask           as time_attn_fwd (causal must be 1; window 0 = unbounded).
 * Query frame a reads frame f iff f <= a and (window == 0 or a - f <= window-1),
 * the predicate of time_attn_fwd, so decoding frame a from a ring filled with
 * frames up to a gives row a of time_attn_fwd over the whole sequence.  The
 * ring must hold every frame read: (q_frame0 + T - 1) - first + 1 <=
 * cache_frames with first = max(0, q_frame0 - window + 1) (0 if window == 0),
 * else BCA_ERR_INVALID_ARG (also for cache_frames <= 0 or q_frame0 < 0).
 * Ownership, alignment, errors and asynchrony as for the other calls. */
int time_attn_decode_fwd(const bca_shape* shape, const bca_mask* mask, const void* q,
                         const void* k_cache, const void* v_cache, int32_t cache_frames,
                         int32_t q_frame0, void* o, float* lse, void* stream);

/* time_attn_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and results as time_attn_bwd, with the workspace
 * taken from a static device array of the library instead of an argument.
 * It calls no hipMalloc, hipFree or allocating library routine.  The array
 * holds 64 MiB per GPU (kept until the process ends), enough for
 * B*T*N*Hq <= 2^24 (query, head) rows or the split partials of up to 128
 * problems.  Where time_attn_bwd would run windowed attention over more
 * than 320 frames as segments whose partials do not fit the array, this
 * call runs the two-kernel backward (Delta rows only), whose results agree
 * with time_attn_bwd's to rounding, not bit for bit.  Shapes whose need
 * still exceeds 64 MiB are refused with BCA_ERR_INVALID_ARG before any
 * launch.  Every call on one GPU uses that
 * GPU's one array: calls that overlap in time on one GPU (other streams,
 * other threads) race and must be serialized by the caller.  Nothing in the
 * array needs to start at any value.  Other arguments, ownership and errors
 * as time_attn_bwd. */
int time_attn_bwd_noalloc(const bca_shape* shape, const bca_mask* mask, const void* q,
                          const void* k, const void* v, const void* o, const float* lse,
                          const void* dout, void* dq, void* dk, void* dv, void* stream);

/* Bytes of device workspace the backward of `op` (BCA_OP_SPACE or
 * BCA_OP_TIME) needs for `shape` on the current device, for any mask.  On
 * the bf16 head_dim-64 path with an attended length (N for space, T for
 * time) of at most 320, every problem (a block or slot and a KV head) is one
 * key block and one kernel forms dQ, dK and dV; it runs one workgroup per
 * problem and compute unit, so the problems pass through the device in
 * rounds.  When there are more problems than compute units and the last
 * round is at most half full, that round's problems each run as two
 * workgroups (one per half of the query rows), whose fp32 dK, dV partials,
 * 2 * ceil(L/16)*16 * 128 * 4 bytes per such problem, go to the workspace and
 * are summed in a fixed order by a second kernel; otherwise this path needs
 * 0 bytes.  With longer attended lengths the backward needs one fp32
 * Delta = rowsum(dO * O) per (query, head), B*T*N*Hq*4 bytes, which its
 * first kernel writes and its second reads; except time attention with a
 * window W whose segments of R positions (the largest multiple of
 * 32 / gcd(G, 32) with R + W - 1 <= 320) hold at least 128: it runs as
 * ceil(T/R) segments per problem, each forming dQ of its rows and writing
 * fp32 dK, dV partials of the keys its rows see, ceil(min(T, R + W - 1)/16)
 * * 16 * 128 * 4 bytes per segment, summed per key by a second kernel.  The
 * query takes no window and returns the most any window needs (segments of
 * 128 positions when T > 320, or Delta when that is larger); a call checks
 * the need of its own mask.  The op is an argument because the attended
 * length depends on it.  Returns 0 for an invalid shape or op. */
size_t bca_bwd_workspace_bytes(int op, const bca_shape* shape);

/* ---- projections beside attention ----
 * Open Dreamer articles (pro.edgex.exchange, fr-FR edition): section
 * "Configuration d'entraînement" -- d_model 1920, 30 query heads over 3 KV
 * heads of width 64; section "Ingénierie de la stabilité", item 3 --
 * parameters in fp32, bf16 for most matmul activations and the attention
 * inputs, fp32 for normalization layers.  All matrices are row-major bf16;
 * weights are the bf16 copies stored (out_features, in_features). */
typedef struct {
  int64_t M;        /* token rows (B*T*N) */
  int32_t d_model;  /* model width; multiple of 8 */
  int32_t Hq, Hkv;  /* query / KV heads */
  int32_t D;        /* head width; multiple of 8 */
} bca_proj_shape;

/* Device workspace rmsnorm_qkv_fwd needs (0 for an invalid shape): a bf16
 * copy of w_qkv with the gain folded in, (Hq + 2 Hkv) * D * d_model * 2 bytes
 * rounded up to a multiple of 256, then M fp32 rstd values (used when the
 * caller passes no rstd). */
size_t bca_qkv_workspace_bytes(const bca_proj_shape* shape);

/* RMS norm then the QKV projection (no biases):
 *   rstd = 1/sqrt(mean_c x[m][c]^2 + eps)                              (fp32)
 *   [q | k | v][m] = (x[m] * rstd[m] * gain) w_qkv^T
 * computed as rstd[m] * (x[m] wg^T) with wg = bf16(w_qkv * gain) formed in
 * the workspace (bf16 operands, fp32 sums, bf16 results).
 *   x      (M, d_model) bf16            gain  (d_model) fp32
 *   w_qkv  ((Hq + 2 Hkv) * D, d_model)  rows: the Q heads, the K heads, the V heads
 *   q      (M, Hq * D), k, v (M, Hkv * D) bf16: with M = B*T*N these are the
 *          (B,T,N,H,D) inputs of the attention calls
 *   rstd   (M) fp32 or NULL (kept for a backward)
 *   workspace at least bca_qkv_workspace_bytes(shape) bytes.
 * Errors as for the attention calls; UNSUPPORTED when d_model or D is not a
 * multiple of 8. */
int rmsnorm_qkv_fwd(const bca_proj_shape* shape, const void* x, const float* gain, float eps,
                    const void* w_qkv, void* q, void* k, void* v, float* rstd, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Output projection with the residual add:
 *   y = residual + o w_o^T    o (M, Hq * D), w_o (d_model, Hq * D),
 *                             residual (M, d_model) or NULL, y (M, d_model). */
int out_proj_fwd(const bca_proj_shape* shape, const void* o, const void* w_o, const void* residual,
                 void* y, void* stream);

/* Static string naming a status code. */
const char* bca_status_string(int status);

/* Detail of the calling thread's last failed call ("" if none). */
const char* bca_last_error(void);

/* BCA_ABI_VERSION of the loaded library. */
int bca_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BCA_H */
