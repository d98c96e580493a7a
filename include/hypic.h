/*
 * hypic.h -- C ABI of the HYPIC linear-layer hot path on one MI355X (gfx950).
 *
 * What the library computes (the pages never print equations; this is the
 * reading the library implements):
 *
 *   Per head a state S in R^{d_k x d_v} follows the gated linear recurrence
 *       S_t = A_t S_{t-1} + beta_t k_t v_t^T ,      S_0 = 0
 *   with the transition family
 *       HYPIC_SCALAR    A_t = alpha_t I               (RetNet / Mamba2 style decay)
 *       HYPIC_DIAGONAL  A_t = diag(alpha_t)           (GLA style gates on the key channels)
 *       HYPIC_GDN       A_t = alpha_t (I - beta_t k_t k_t^T)   (gated delta rule; DeltaNet = alpha 1)
 *       HYPIC_KDA       A_t = (I - beta_t k_t k_t^T) diag(alpha_t)   (one gate per key channel)
 *   For a segment C of n tokens its record is the cumulative transition operator
 *   T_C = A_n ... A_1 and the zero-initial terminal state S(C|0) = S_n, so that
 *   a start state S_0 maps to T_C S_0 + S(C|0).  Segments are then composed in
 *   prompt order, S = T_C2 S(C1) + S(C2), which equals the recurrence run over
 *   the concatenation.
 *
 *   Sources: "HYPIC: Cache Acceleration for Hybrid Attention Models"
 *   (agihunt.info), "Core Approach" (cache T_C beside the zero-initial terminal
 *   state; constant-time combination on reuse); "Cut First-Token Latency by
 *   3.25x: Introducing HYPIC ..." (besthub.dev), paragraph 4 (store the pair at
 *   first prefill, compose T_C2*S(C1)+S(C2); the family list; the convolution
 *   state warm-up patch); "Hypic: Position-Independent KV Caching for
 *   Hybrid-Attention LLM Serving" (podcast companion page), "The transition
 *   operator: compose, don't add" and "Family comparison: scalar -> diagonal ->
 *   dense"; its reference 7 (Gated Delta Networks) for the GDN transition.
 *
 * Stored record (exact factorisation, not an approximation).  The scalar gate
 * commutes with everything, so T_C = e^{ell} P with ell = sum_t log alpha_t
 * and P = prod_{t=n..1} (I - beta_t k_t k_t^T).  A pool record per head is
 *       log_scale  ell         1 float (d_k floats for HYPIC_DIAGONAL)
 *       P          d_k x d_k   fp32, row-major (HYPIC_GDN; for HYPIC_KDA, whose gates do not
 *                  factor out, P = T_C itself and ell = 0; P = I otherwise)
 *       S          d_k x d_v   fp32, row-major
 * Keeping ell apart keeps T_C inside fp32 range: e^{ell} of a 2048-token
 * segment is far below the smallest fp32 normal at typical decay rates.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is DEVICE memory owned by the caller; the library
 *     never allocates, frees or retains a pointer past the call.  Descriptor
 *     structs are host memory read only during the call.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream).  No host synchronisation happens inside.
 *   - The return code reports synchronous argument validation and launch
 *     errors only; on any error nothing is launched.  Validation happens
 *     before any HIP call.
 *   - Data-dependent errors (slot ids, offsets) are OR-ed into the device word
 *     *err_flag (HYPIC_EFLAG_*), when err_flag is not NULL; the output they
 *     concern is filled with NaN (when it exists) and every other output is
 *     computed normally.  The caller clears *err_flag.
 *   - Inputs are never written; outputs are overwritten in full; inputs and
 *     outputs must not alias.  There is no global mutable state: concurrent
 *     calls on different streams are safe when their outputs do not overlap.
 *   - Supported head sizes: d_k, d_v in {64, 128}.
 */
#ifndef HYPIC_H
#define HYPIC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HYPIC_ABI_VERSION 1

typedef enum {
    HYPIC_OK = 0,
    HYPIC_ERR_INVALID_ARG = 1,   /* NULL required pointer, negative size, family/shape mismatch */
    HYPIC_ERR_UNSUPPORTED = 2,   /* d_k or d_v not in {64,128}, unknown dtype, family or activation */
    HYPIC_ERR_HIP = 3            /* the kernel launch failed (hipGetLastError) */
} hypic_status;

typedef enum { HYPIC_SCALAR = 0, HYPIC_DIAGONAL = 1, HYPIC_GDN = 2, HYPIC_KDA = 3 } hypic_family;
typedef enum { HYPIC_F32 = 0, HYPIC_BF16 = 1 } hypic_dtype;

#define HYPIC_EFLAG_SLOT_OUT_OF_RANGE 0x1u   /* a slot id outside [0, num_slots) */
#define HYPIC_EFLAG_BAD_OFFSETS       0x2u   /* decreasing offsets, or an offset outside [0, num_tokens] */

/*
 * Segment pool: caller-owned device memory holding one record per (slot, head).
 *   log_scale  [num_slots][H] fp32, or [num_slots][H][d_k] for HYPIC_DIAGONAL
 *   P          [num_slots][H][d_k][d_k] fp32, HYPIC_GDN and HYPIC_KDA only (NULL otherwise)
 *   S          [num_slots][H][d_k][d_v] fp32
 * All three are dense and row-major.
 */
typedef struct hypic_pool {
    int32_t family;       /* hypic_family */
    int32_t num_heads;    /* H */
    int32_t d_k, d_v;
    int64_t num_slots;
    float *log_scale;
    float *P;
    float *S;
} hypic_pool;

/*
 * A packed stream of segments (device pointers; strides in ELEMENTS, the
 * innermost channel stride is 1).
 *   token t, head h:  k[t*k_stride_t + h*k_stride_h + i]   i < d_k   (kv_dtype)
 *                     v[t*v_stride_t + h*v_stride_h + j]   j < d_v   (kv_dtype)
 *                     beta[t*beta_stride_t + h*beta_stride_h]        (fp32; NULL means beta = 1)
 *                     log_alpha[t*la_stride_t + h*la_stride_h (+ i for HYPIC_DIAGONAL, HYPIC_KDA)]
 *                                                          (fp32, log of the decay; NULL means 0)
 *   la_stride_t = 0 gives a per-head constant decay (RetNet).
 *   Segment s is tokens [seg_offsets[s], seg_offsets[s+1]) (device int64,
 *   num_segments+1 entries, non-decreasing, inside [0, num_tokens]).
 *   A segment may be empty (identity record) and needs no particular length.
 */
typedef struct hypic_segments {
    int32_t family;       /* hypic_family; must equal the pool's */
    int32_t num_heads;
    int32_t d_k, d_v;
    int32_t num_segments;
    int32_t kv_dtype;     /* hypic_dtype of k and v */
    int64_t num_tokens;   /* rows of the packed stream, bound for the offsets */
    const int64_t *seg_offsets;
    const void *k;          int64_t k_stride_t, k_stride_h;
    const void *v;          int64_t v_stride_t, v_stride_h;
    const float *beta;      int64_t beta_stride_t, beta_stride_h;
    const float *log_alpha; int64_t la_stride_t, la_stride_h;
} hypic_segments;

/*
 * hypic_build_segment -- build the record (ell, P, S) of every segment and head
 * of `in` and write it to pool slot dst_slots[s] (device int32, one per
 * segment; distinct).  Source: besthub article, paragraph 4 (the pair
 * (T_C, S(C|0)) is stored during the first prefill); agihunt summary, "Core
 * Approach" (the segment-cumulative transition operator T_C).
 *
 * Error behaviour: a dst slot outside [0, num_slots) sets
 * HYPIC_EFLAG_SLOT_OUT_OF_RANGE and writes nothing for that segment; bad
 * offsets set HYPIC_EFLAG_BAD_OFFSETS and fill the segment's record with NaN.
 * NaN or Inf inputs propagate into the affected record.
 *
 * HYPIC_KDA at d_k = d_v = 128 runs in 32-token chunks on the fp32 matrix
 * cores; a chunk in which some channel's gate product over seven tokens falls
 * below about e^-69 is applied token by token instead (same result, slower).
 * Other KDA shapes run token by token throughout.
 */
hypic_status hypic_build_segment(const hypic_segments *in, const hypic_pool *pool,
                                 const int32_t *dst_slots, uint32_t *err_flag, void *stream);

/*
 * hypic_prefill_segment -- the chunked prefill forward of every segment and head of
 * `in`, each from a zero state at the segment's first token, read out at every token:
 *       o_t = S_t^T q_t        (S_t: the head's state right after token t's update)
 * and, when pool is not NULL, the segment's record (ell, P, S) written to pool slot
 * dst_slots[s] exactly as hypic_build_segment defines it.  Source: besthub article,
 * paragraph 7 (the one-time construction of (T_C, S) next to the ordinary prefill
 * forward) and paragraph 4 (the record); podcast page, reference 7 (the GDN
 * recurrence whose states are read out).
 *
 *   q         [N][H][d_k] in kv_dtype: q[t*q_stride_t + h*q_stride_h + i]
 *   o         [N][H][d_v] in o_dtype (HYPIC_F32 or HYPIC_BF16):
 *             o[t*o_stride_t + h*o_stride_h + j]; written for every token of every
 *             segment and nowhere else (segments must not overlap).  o = NULL (q
 *             ignored): the records alone, exactly as hypic_build_segment.
 *   pool, dst_slots   as hypic_build_segment, or NULL for the outputs alone.
 * At least one of o and pool.  GDN with bf16 k, v and q at d_k = d_v = 128, rows
 * 16-byte aligned and strides multiples of 8 elements; anything else returns
 * HYPIC_ERR_UNSUPPORTED (nothing launched).
 *
 * Error behaviour: the flags of hypic_build_segment.  A dst slot out of range: nothing
 * of that segment is written (neither its record nor its outputs).  Bad offsets: its
 * record (when built) is filled with NaN and none of its outputs is written (there
 * is no token range to write).  Every other segment is computed normally.
 */
hypic_status hypic_prefill_segment(const hypic_segments *in, const void *q, int64_t q_stride_t,
                                   int64_t q_stride_h, void *o, int64_t o_stride_t, int64_t o_stride_h,
                                   int32_t o_dtype, const hypic_pool *pool, const int32_t *dst_slots,
                                   uint32_t *err_flag, void *stream);

/*
 * hypic_compose_chain -- for every request r and head h, fold the pool records
 * chain_slots[chain_offsets[r] .. chain_offsets[r+1]) in prompt order:
 *       S <- T_i S + S_i = e^{ell_i} (P_i S) + S_i
 * starting from init_S[r][h] (NULL = zero).  Source: besthub article,
 * paragraph 4 (reuse composes T_C2*S(C1)+S(C2) in constant time); podcast
 * page, "Composition law, step by step".
 *
 *   chain_offsets  device int64 [num_requests+1], non-decreasing from 0
 *   chain_slots    device int32, slot ids; repeats allowed; an empty chain
 *                  yields init_S (or 0)
 *   init_S         [R][H][d_k][d_v] fp32 or NULL
 *   out_S          [R][H][d_k][d_v] fp32 (required)
 *   out_log_scale  [R][H] ([R][H][d_k] diagonal) fp32 or NULL: sum of ell_i (plus the
 *                  renormalisation of out_P, when that is asked for)
 *   out_P          [R][H][d_k][d_k] fp32 or NULL (GDN, KDA): P_m ... P_1 up to a power of
 *                  two that out_log_scale carries; needs out_log_scale (else
 *                  HYPIC_ERR_INVALID_ARG).  A product of contracting records shrinks
 *                  toward the fp32 subnormals (a GDN record's P by about e^-4 per 2048
 *                  tokens at unit keys); below 2^-32 the product is scaled back by an
 *                  exact power of two 2^s and s ln 2 is taken off out_log_scale, so
 *                  that T = e^{out_log_scale} out_P holds throughout
 *   (out_log_scale, out_P, out_S) is the record of the concatenated chain formed from the
 *   chain's records: out_P is their product up to fp32 rounding (about 16 bits per
 *   product on the matrix cores), so its error against the operator of the
 *   concatenated tokens is the records' own error compounded over the chain, about
 *   sqrt(m) times a record's for m records with independent rounding.
 *
 * Error behaviour: a slot id outside [0, num_slots) sets
 * HYPIC_EFLAG_SLOT_OUT_OF_RANGE, bad chain offsets set HYPIC_EFLAG_BAD_OFFSETS;
 * in both cases that request's outputs are filled with NaN.
 */
hypic_status hypic_compose_chain(const hypic_pool *pool, int32_t num_requests,
                                 const int64_t *chain_offsets, const int32_t *chain_slots,
                                 int64_t num_chain_slots,
                                 const float *init_S, float *out_S, float *out_log_scale,
                                 float *out_P, uint32_t *err_flag, void *stream);

/*
 * hypic_compose_chain_heads -- hypic_compose_chain where chain entry c first
 * applies a few tokens to the state, then folds its record:
 *       for t in [head_offsets[c], head_offsets[c+1]):
 *           S <- alpha_t (S - beta_t k_t (k_t^T S)) + beta_t k_t v_t^T   (alpha_t = e^{log_alpha_t})
 *       S <- e^{ell_i} (P_i S) + S_i
 * and out_log_scale adds the tokens' log alpha.  For conv variants (besthub
 * article, paragraph 4: the convolution state warm-up): the tokens are a reused
 * segment's first K-1, whose keys and values the warmed conv produced
 * (hypic_conv_kv), and the record is the segment's suffix, so the chain equals
 * the recurrence over the concatenated request without a record per head.
 *
 *   head_offsets   device int64 [num_chain_slots+1], non-decreasing, inside
 *                  [0, num_head_tokens], at most 8 tokens per entry
 *   head_k         [T][H][d_k] fp32;  head_v [T][H][d_v] fp32
 *   head_beta, head_log_alpha   [T][H] fp32           (T = num_head_tokens)
 * GDN pools with d_k = d_v = 128 only (else HYPIC_ERR_UNSUPPORTED); no composed
 * operator.  num_head_tokens = 0 (all four head pointers NULL) is the plain chain.
 * Error behaviour as hypic_compose_chain; malformed head offsets (or more than 8
 * tokens at an entry) set HYPIC_EFLAG_BAD_OFFSETS and NaN-fill that request.
 */
hypic_status hypic_compose_chain_heads(const hypic_pool *pool, int32_t num_requests,
                                       const int64_t *chain_offsets, const int32_t *chain_slots,
                                       int64_t num_chain_slots, const int64_t *head_offsets,
                                       int64_t num_head_tokens, const float *head_k, const float *head_v,
                                       const float *head_beta, const float *head_log_alpha,
                                       const float *init_S, float *out_S, float *out_log_scale,
                                       uint32_t *err_flag, void *stream);

/*
 * hypic_conv_warmup -- convolution state warm-up at segment boundaries
 * (besthub article, paragraph 4).  A causal depthwise conv of kernel size K
 * runs before the recurrence in conv variants; a segment prefilled on its own
 * saw a zero history for its first K-1 tokens.  At boundary b the warm-up
 * recomputes those outputs with the previous segment's last K-1 raw inputs as
 * the conv state:
 *       x_bar = [tail_b (K-1 rows) ; head_b (K-1 rows)]
 *       out[b][t][c] = act( bias[c] + sum_{j<K} w[c][j] * x_bar[t+j][c] ),  t < K-1
 * (w[c][K-1] multiplies the current token).  act: 0 identity, 1 SiLU.
 *
 *   tails       [num_tails][K-1][C] raw inputs (x_dtype), rows in stream order
 *   tail_index  device int32 [B] or NULL (boundary b uses tails[b])
 *   heads       [num_heads][K-1][C] raw inputs (x_dtype)
 *   head_index  device int32 [B] or NULL (boundary b uses heads[b])
 *   weight      [C][K] fp32;  bias [C] fp32 or NULL
 *   out         [B][K-1][C] fp32
 *   2 <= K <= 8.
 * Error behaviour: an index outside its table sets
 * HYPIC_EFLAG_SLOT_OUT_OF_RANGE and fills that boundary's output with NaN.
 */
hypic_status hypic_conv_warmup(int32_t num_boundaries, int32_t channels, int32_t kernel_size,
                               int32_t x_dtype,
                               const void *tails, int64_t num_tails, const int32_t *tail_index,
                               const void *heads, int64_t num_heads, const int32_t *head_index,
                               const float *weight, const float *bias, int32_t activation,
                               float *out, uint32_t *err_flag, void *stream);

/*
 * hypic_conv_kv -- keys and values of chosen tokens of a conv variant, from raw
 * inputs (besthub article, paragraph 4: the convolution state warm-up that keeps
 * reused segments aligned).  In a conv variant a causal depthwise conv of kernel
 * size K and an activation run over time before the recurrence, and the keys are
 * L2-normalised per head.  For output token t:
 *       y[c]    = act( bias[c] + sum_{j<K} w[c][j] * x[window[t][j]][c] ),  C = H (d_k + d_v)
 *       k[t][h] = y[h d_k .. h d_k + d_k) / sqrt(sum of squares + 1e-6)     (normalize_k != 0)
 *       v[t][h] = y[H d_k + h d_v .. + d_v)
 * (w[c][K-1] multiplies window[t][K-1], the token itself).  With the window rows
 * of a segment's own earlier tokens this is its first prefill; with the previous
 * segment's last raw inputs in the window it is the warm-up of a reused
 * segment's first K-1 tokens, whose keys and values then feed a short record
 * (hypic_build_segment) composed between the two segments' records.
 *
 *   x            [num_rows][C] raw inputs (x_dtype), row-major
 *   window       device int32 [num_tokens][K]: rows of x, -1 = a zero row
 *   weight       [C][K] fp32;  bias [C] fp32 or NULL;  act: 0 identity, 1 SiLU
 *   k_out        [num_tokens][H][d_k] (out_dtype);  v_out [num_tokens][H][d_v]
 *   src_token    device int32 [num_tokens] or NULL: when given, beta_out[t][h] =
 *                beta[src_token[t]][h] (1 when beta is NULL) and la_out[t][h] =
 *                log_alpha[src_token[t]][h] (0 when NULL); beta, log_alpha
 *                [num_src_tokens][H] fp32; beta_out, la_out [num_tokens][H] fp32
 *   1 <= K <= 8, H (d_k + d_v) <= 16384.
 * Error behaviour: a window row outside [-1, num_rows) or a src_token outside
 * [0, num_src_tokens) sets HYPIC_EFLAG_SLOT_OUT_OF_RANGE and fills that token's
 * outputs with NaN.
 */
hypic_status hypic_conv_kv(int32_t num_tokens, int32_t num_heads, int32_t d_k, int32_t d_v, int32_t kernel_size,
                           int32_t x_dtype, const void *x, int64_t num_rows, const int32_t *window,
                           const float *weight, const float *bias, int32_t activation, int32_t normalize_k,
                           int32_t out_dtype, void *k_out, void *v_out,
                           const int32_t *src_token, int64_t num_src_tokens, const float *beta,
                           const float *log_alpha, float *beta_out, float *la_out,
                           uint32_t *err_flag, void *stream);

/* Human-readable name of a status code (static storage). */
const char *hypic_status_string(int32_t status);

/* HYPIC_ABI_VERSION of the built library. */
int32_t hypic_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HYPIC_H */
