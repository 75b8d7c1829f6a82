/*
 * attn.h -- C ABI of the fused, I/O-aware forward pass of exact scaled
 * dot-product attention on AMD Instinct MI355X (gfx950), with its backward
 * pass, grouped-query variants of both, decode over a key/value cache, and
 * the unfused (materialised) forward it is measured against.
 *
 * For every (batch b, head h) the library computes, for queries Q, keys K
 * and values V of shape T x d,
 *
 *   S   = scale * Q K^T                 scores, rows = queries, cols = keys
 *   S_ij = -inf for j > i               only when causal = 1
 *   P   = row softmax of S              exp(S_ij) / sum_j exp(S_ij)
 *   O   = P V                           T x d output
 *   LSE_i = ln sum_j exp(S_ij)          natural-log "exponential sum"
 *
 * as defined on "Attention Mechanism: Computation & Memory Patterns"
 * (section 1, the attention equation and its three steps) and "Why Attention
 * Is Difficult to Optimize" ("The Attention Computation Flow", Figure 1:
 * scale, then causal mask, then softmax, then PV).  The T x T matrices S and
 * P never reach device memory: the kernel walks key/value tiles with an
 * online softmax (running max, running normaliser, rescaled fp32 output
 * accumulator), as described on "Attention Mechanism: Computation & Memory
 * Patterns" (section 3, tiling and online softmax) and "FlashAttention --
 * avoid writing the giant intermediate" ("Tiling and an incremental
 * normalization").  LSE is an extra per-row output the pages do not define;
 * it is the natural log of the row's exponential sum of scaled, masked
 * scores.
 *
 * Layout.  q, k, v, o are contiguous [B][H][T][d] arrays (d innermost,
 * element (b,h,t,c) at ((b*H + h)*T + t)*d + c); lse is a contiguous
 * [B][H][T] float array.  All pointers are device pointers.
 *
 * Ownership.  The caller owns every buffer.  The library allocates, frees
 * and keeps no device memory; the forward uses no workspace, the backward,
 * the decode and the materialised forward caller-owned ones.  It holds no
 * mutable state other than a per-device cache of the architecture check
 * and CU count, and may be called from several host threads.
 *
 * Asynchrony.  Calls enqueue their kernels (one for the forward, three for
 * the backward and the materialised forward, one or two for the decode) on
 * `stream` (NULL = the null stream) and return; they never synchronise.
 *
 * Errors.  Arguments are validated on the host before any HIP call; on a
 * validation error nothing is launched and the outputs are untouched.  An
 * unsupported head dimension or device is an error, never a fallback.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a pointer is NULL for a non-empty problem      */
  ATTN_ERR_SHAPE = 2,       /* sizes negative, inconsistent or over limits    */
  ATTN_ERR_UNSUPPORTED = 3, /* head dimension d is not 64 or 128              */
  ATTN_ERR_SCALE = 4,       /* scale is NaN or infinite                       */
  ATTN_ERR_ALIGN = 5,       /* q/k/v/o not 16-byte or lse not 4-byte aligned  */
  ATTN_ERR_ARG = 6,         /* causal not 0/1, or an output overlaps a buffer */
  ATTN_ERR_DEVICE = 7,      /* the current device is not gfx950               */
  ATTN_ERR_LAUNCH = 8,      /* the HIP runtime reported an error at launch    */
  ATTN_ERR_WORKSPACE = 9    /* the workspace is missing or too small          */
} attn_status;

/*
 * bfloat16 forward.  q, k, v: const __hip_bfloat16 [B][H][T][d]; o:
 * __hip_bfloat16 [B][H][T][d], written with round-to-nearest-even; lse:
 * float [B][H][T].  Scores and all softmax state are fp32; both
 * contractions run on bf16 MFMA with fp32 accumulation, and P is rounded to
 * bf16 (nearest-even) before the PV contraction.
 *   B, H, T >= 0 (B*H*T == 0: nothing to do, ATTN_OK, pointers unchecked);
 *          (T + 256) * d * sizeof(element) < 2^31 (one head under 2 GiB) and
 *          B*H*ceil(T/128) < 2^31;
 *   d in {64, 128};
 *   causal: 0 = full attention, 1 = key j visible to query i iff j <= i;
 *   scale: any finite multiplier of Q K^T (usually 1/sqrt(d)); it is applied
 *          to the fp32 scores, never folded into bf16 inputs.
 * Outputs must not overlap each other or any input.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o,
                     float* lse, int64_t B, int64_t H, int64_t T, int64_t d,
                     int causal, float scale, hipStream_t stream);

/*
 * Grouped-query forward ("FlashAttention -- avoid writing the giant
 * intermediate", closing note: grouped-query attention changes the head
 * structure of the stored keys and values).  H query heads share H_kv
 * key/value heads, G = H / H_kv query heads per key/value head: query head h
 * reads key/value head h / G (consecutive query heads form a group).
 * q, o: [B][H][T][d]; k, v: [B][H_kv][T][d]; lse: [B][H][T].  H_kv >= 1
 * must divide H (H_kv = H is attn_fwd; H_kv = 1 is multi-query attention);
 * otherwise ATTN_ERR_SHAPE.  Everything else as for attn_fwd.  Workgroups of
 * one group are placed on one XCD when B*H_kv is a multiple of 8, so the
 * group's K/V tiles are fetched into one L2.
 */
attn_status attn_fwd_gqa(const void* q, const void* k, const void* v, void* o,
                         float* lse, int64_t B, int64_t H, int64_t H_kv,
                         int64_t T, int64_t d, int causal, float scale,
                         hipStream_t stream);

/*
 * float32 forward: the same operation ("Attention Mechanism: Computation &
 * Memory Patterns", section 1; "Why Attention Is Difficult to Optimize",
 * "The Attention Computation Flow") and the same contract as attn_fwd, with
 * float elements in q, k, v, o.  Both contractions use fp32 MFMA (no
 * reduced-precision inputs); P stays fp32, so one normaliser serves O and
 * LSE.  A second exported symbol rather than a dtype argument, because the
 * bf16 signature above is fixed; both are instances of one kernel design.
 */
attn_status attn_fwd_f32(const float* q, const float* k, const float* v,
                         float* o, float* lse, int64_t B, int64_t H,
                         int64_t T, int64_t d, int causal, float scale,
                         hipStream_t stream);

/*
 * bfloat16 backward pass ("Attention Mechanism: Computation & Memory
 * Patterns", section 4 and its conclusion: the pass recomputes the scores
 * the forward did not store).  For the forward above and an upstream
 * gradient dO of O it computes, per (batch, head),
 *
 *   dV = P^T dO
 *   dS_ij = P_ij (dP_ij - Delta_i),  dP = dO V^T,  Delta_i = sum_c dO_ic O_ic
 *   dQ = scale dS K,   dK = scale dS^T Q
 *
 * with P_ij = exp(S_ij - LSE_i) rebuilt tile by tile from q, k and the
 * forward's lse (masked entries are 0, so the causal mask passes no
 * gradient).  No T x T matrix is stored.
 *   q, k, v, o, dout: const __hip_bfloat16 [B][H][T][d] (o and lse as the
 *          forward wrote them for the same q, k, v, causal and scale);
 *   lse:   const float [B][H][T];
 *   dq, dk, dv: __hip_bfloat16 [B][H][T][d], written (nearest-even);
 *   ws:    float workspace of 2*B*H*T elements, owned by the caller.  On
 *          return ws[0 .. B*H*T) holds -Delta and ws[B*H*T .. 2*B*H*T)
 *          holds -lse / scale when |scale| >= 2^-32, else -lse * log2(e),
 *          both [B][H][T] (the values the kernels start their score and dP
 *          accumulators from).
 *   B, H, T, d, causal, scale: as for attn_fwd.
 * S, P, dP, dS, Delta are fp32; P and dS are rounded to bf16 (nearest-even)
 * as inputs of the bf16 MFMA contractions, which accumulate in fp32.  Three
 * kernels are enqueued on `stream` in order (row statistics, dK/dV, dQ);
 * every output element is written exactly once, so results do not depend on
 * scheduling.  Pointers: 16-byte aligned (lse, ws: 4-byte).  dq, dk, dv and
 * ws must not overlap each other or any input.  Errors as for attn_fwd.
 */
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk,
                     void* dv, float* ws, int64_t B, int64_t H, int64_t T,
                     int64_t d, int causal, float scale, hipStream_t stream);

/*
 * Grouped-query backward: the gradient of attn_fwd_gqa.  k, v, dk, dv are
 * [B][H_kv][T][d]; dK and dV of a key/value head sum the contributions of
 * its G query heads (accumulated in registers by one workgroup, no
 * atomics).  Everything else as for attn_bwd (ws: 2*B*H*T floats).
 */
attn_status attn_bwd_gqa(const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse,
                         void* dq, void* dk, void* dv, float* ws, int64_t B,
                         int64_t H, int64_t H_kv, int64_t T, int64_t d,
                         int causal, float scale, hipStream_t stream);

/*
 * Name of kernel `which` (0 = row statistics, 1 = dK/dV, 2 = dQ) that
 * attn_bwd launches for head dimension d and the causal flag, e.g.
 * "attn_bwd_dkdv_bf16_d128_causal_bk256_bq64_w8".  NULL if unsupported.
 */
const char* attn_bwd_kernel_name(int64_t d, int causal, int which);

/*
 * Name of kernel `which` (as attn_bwd_kernel_name) that attn_bwd_gqa
 * launches for these sizes on the current device, to inspect the instance
 * actually selected ("FlashAttention -- avoid writing the giant
 * intermediate", "Apply it at the right layer").  The dK/dV kernel takes
 * 256-key workgroups of 8 waves, or, when B * H_kv * ceil(T / 256) is below
 * the device's CU count (with causal = 1, below twice the CU count, or at
 * most four times it with T <= 4096), 128-key workgroups of 8 waves, two per
 * 32 keys
 * ("attn_bwd_dkdv_bf16_d128_causal_bk128_bq64_w8"); the dQ kernel takes
 * 128-query workgroups of 4 waves, or, when B * H * ceil(T / 128) is below
 * twice the CU count (with causal = 1, at most twice), of 8 waves, two per
 * 32 queries
 * ("attn_bwd_dq_bf16_d128_causal_bq128_bk64_w8").  NULL for unsupported or
 * non-positive sizes, or when the current device is not a gfx950.
 */
const char* attn_bwd_kernel_name_for(int64_t B, int64_t H, int64_t H_kv, int64_t T, int64_t d,
                                     int causal, int which);

/*
 * Decode: Tq new queries per head over a key/value cache ("FlashAttention --
 * avoid writing the giant intermediate": short-input decode against the
 * stored key/value state, as opposed to long-input prefill).  The queries
 * are the last Tq positions of the cached sequence: query i sits at
 * position Tk - Tq + i and, with causal = 1, sees keys j <= Tk - Tq + i
 * (without the mask, all Tk keys).  O and LSE are defined as for the
 * forward.
 *   q, o:  __hip_bfloat16 [B][H][Tq][d];  lse: float [B][H][Tq];
 *   k, v:  const __hip_bfloat16 caches [B][H_kv][Tk_cap][d] of which rows
 *          0 .. Tk-1 of each head are valid (rows >= Tk are never read);
 *   H_kv divides H, query head h reads key/value head h / (H / H_kv);
 *   Tq * (H / H_kv) query rows per key/value head, at most 2^30: up to
 *          32 of them share one workgroup and one read of the keys, more
 *          take one workgroup per 32 rows (many new queries appended to a
 *          cache, a prefill in chunks, run the same way; under the causal
 *          mask a workgroup reads only the keys its rows can see; with
 *          at least 256 of them and B * H * ceil(Tq / 128) at least the
 *          device's CU count, the forward kernel runs them instead, as one
 *          kernel with no workspace);
 *          1 <= Tk <= Tk_cap, and Tk >= Tq when causal (ATTN_ERR_SHAPE
 *          otherwise);
 *   ws, ws_bytes: caller-owned device workspace of at least
 *          attn_decode_workspace_bytes(B, H, H_kv, Tq, Tk, d) bytes,
 *          16-byte aligned (may be NULL when that is 0), overwritten.  Too
 *          small: ATTN_ERR_WORKSPACE.
 * The keys are split into attn_decode_splits(B, H, H_kv, Tq, Tk) consecutive
 * ranges, one workgroup each, whose partial results (normalised output and
 * LSE per query row, fp32, in ws) a second kernel merges as
 * LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.  The query heads
 * of one key/value head are processed together, so the cache is read once
 * per group.  Two kernels are enqueued (one when there is a single split).
 * Other arguments and errors as for attn_fwd.
 */
attn_status attn_decode(const void* q, const void* k, const void* v, void* o,
                        float* lse, void* ws, int64_t ws_bytes, int64_t B,
                        int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk,
                        int64_t Tk_cap, int64_t d, int causal, float scale,
                        hipStream_t stream);

/*
 * Decode without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops or harnesses that forbid allocation).  Same computation,
 * kernels, arguments and errors as attn_decode, except that the split
 * partial results go to a scratch buffer of ATTN_DECODE_NOALLOC_MAX_BYTES
 * bytes that the library holds in device memory, one per GPU it runs on,
 * until the process ends.  Problems whose attn_decode_workspace_bytes(...)
 * exceeds that size are rejected with ATTN_ERR_WORKSPACE before anything is
 * enqueued: splits x B x H x Tq may be at most 8 MiB / (4 (d + 1)), 16,256
 * at d = 128 (16 sequences x 32 query heads x 1 query over 32768 keys take
 * 4 splits and 264 KiB; a grid of at least 256 workgroups without splits
 * needs none).  The buffer is fully rewritten by each call before
 * it is read, so nothing needs clearing; but every call on one GPU shares
 * it: calls that can overlap on one GPU (different streams, or host threads
 * without ordering) race and must be serialised by the caller.  The first
 * call on each device looks up the buffer's address (no allocation) with
 * that device current.
 */
#define ATTN_DECODE_NOALLOC_MAX_BYTES (8 << 20)

attn_status attn_decode_noalloc(const void* q, const void* k, const void* v,
                                void* o, float* lse, int64_t B, int64_t H,
                                int64_t H_kv, int64_t Tq, int64_t Tk,
                                int64_t Tk_cap, int64_t d, int causal,
                                float scale, hipStream_t stream);

/* Workspace bytes attn_decode needs for these sizes (0 if none, or if the
 * sizes are invalid). */
int64_t attn_decode_workspace_bytes(int64_t B, int64_t H, int64_t H_kv,
                                    int64_t Tq, int64_t Tk, int64_t d);

/* Number of key ranges attn_decode splits each key/value head into
 * (0 if the sizes are invalid). */
int64_t attn_decode_splits(int64_t B, int64_t H, int64_t H_kv, int64_t Tq,
                           int64_t Tk);

/*
 * Name of the kernel attn_decode launches first for these sizes on the
 * current device: "attn_decode_bf16_d128_causal_w4_blk32" (and d64 / full
 * variants) for the split-key kernel, or the forward instance (as
 * attn_fwd_kernel_name_for names them) when the new queries are many enough
 * for the forward kernel to run over the cache.  Lets a caller inspect the
 * route actually taken for a decode or prefill chunk ("FlashAttention --
 * avoid writing the giant intermediate", "Apply it at the right layer":
 * check which backend was selected, and measure decode separately from
 * prefill).  NULL if the sizes are invalid or the device is not a gfx950.
 */
const char* attn_decode_kernel_name_for(int64_t B, int64_t H, int64_t H_kv,
                                        int64_t Tq, int64_t Tk, int64_t d,
                                        int causal);

/*
 * Materialised forward: the unfused three-kernel path that writes the T x T
 * score matrix S (fp32) and probability matrix P (bf16) to device memory and
 * reads them back ("Why Attention Is Difficult to Optimize", Figure 2: the
 * naive sequence of separate kernels, each round-tripping through HBM), for
 * measuring the time and traffic the fused forward avoids.  Same inputs,
 * outputs and definitions as attn_fwd (O = P V with P rounded to bf16, LSE
 * natural log).
 *   s_buf: float [B][H][T][T] scratch, p_buf: __hip_bfloat16 [B][H][T][T]
 *          scratch, both caller-owned and overwritten; under the causal mask
 *          only the 64-key tiles at or below the diagonal of each 128-query
 *          block are written and read;
 *   T must be a multiple of 128 and at most 32768 (ATTN_ERR_UNSUPPORTED /
 *          ATTN_ERR_SHAPE); d in {64, 128}.
 * Three kernels are enqueued on `stream` (scores, row softmax, P V).
 */
attn_status attn_fwd_materialized(const void* q, const void* k, const void* v,
                                  void* o, float* lse, float* s_buf,
                                  void* p_buf, int64_t B, int64_t H, int64_t T,
                                  int64_t d, int causal, float scale,
                                  hipStream_t stream);

/*
 * Static description of a status code (never NULL).  Every unsupported
 * request is reported by a code, never served by another path
 * ("FlashAttention -- avoid writing the giant intermediate", "Apply it at
 * the right layer": a requested option may be unsupported or fall back, so
 * check what ran).
 */
const char* attn_status_string(attn_status s);

/*
 * Name of the kernel instance attn_fwd (is_f32 = 0) or attn_fwd_f32
 * (is_f32 = 1) launches for head dimension d and the causal flag, e.g.
 * "attn_fwd_bf16_d128_causal_br256_bc64_w8", so that a caller can log which
 * kernel ran ("FlashAttention -- avoid writing the giant intermediate",
 * "Apply it at the right layer": inspect the backend actually selected).
 * The mask is part of the name because masked and unmasked problems run
 * different instances.  For bf16 this is the instance of grids with at least one
 * 256-row workgroup per CU (smaller grids: see attn_fwd_kernel_name_for).  NULL if the combination
 * is unsupported.
 */
const char* attn_kernel_name(int is_f32, int64_t d, int causal);

/*
 * Name of the kernel instance attn_fwd / attn_fwd_gqa launch for these sizes
 * on the current device (B * H query heads):
 *   - the row-chunk kernel (32 query rows per workgroup, their keys split
 *     over 4 waves, e.g. "attn_fwd_rows_bf16_d64_causal_br32_bc32_w4") when
 *     B * H * ceil(T / 128) * (d / 64) is at most the device's CU count;
 *   - else the 4-wave instance (128 rows, e.g.
 *     "attn_fwd_bf16_d128_causal_br128_bc64_w4") when B * H * ceil(T / 256)
 *     is below the CU count, or equal to it with causal = 1 and T >= 2048
 *     (d = 128) or T >= 4096 (d = 64): one round of blocks whose work the
 *     mask makes unequal;
 *   - else the 8-wave instance (256 query rows per workgroup).
 * NULL if the sizes are unsupported or the current device is not a gfx950.
 */
const char* attn_fwd_kernel_name_for(int64_t B, int64_t H, int64_t T,
                                     int64_t d, int causal);

/*
 * Name of the kernel instance attn_fwd_f32 launches for these sizes on the
 * current device: at d = 64, when B * H * ceil(T / 128) is below the
 * device's CU count, the row-chunk kernel (32 query rows per workgroup,
 * their keys split over 4 waves, "attn_fwd_f32_rows_d64_causal_br32_bc32_w4"
 * or "..._full_..."); otherwise the instance attn_kernel_name(1, d, causal)
 * names.  NULL if the sizes are unsupported or the device is not a gfx950.
 */
const char* attn_fwd_f32_kernel_name_for(int64_t B, int64_t H, int64_t T,
                                         int64_t d, int causal);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
