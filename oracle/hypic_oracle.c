/*
 * hypic_oracle.c -- plain fp64 CPU oracle for the HYPIC linear-layer segment
 * cache: segment records (T_C, S(C|0)), their composition, and the causal
 * short-conv used by the convolution state warm-up.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this library.  It shares no code, header, table
 * or helper with the GPU library, and the GPU library never calls it.
 *
 * Sources (the pages this follows):
 *  - "HYPIC: Cache Acceleration for Hybrid Attention Models" (agihunt.info),
 *    section "Core Approach": linear layers cache the segment-cumulative
 *    transition operator T_C next to the zero-initial terminal state, and
 *    combine states in constant time on reuse.
 *  - "Cut First-Token Latency by 3.25x: Introducing HYPIC ..." (besthub.dev),
 *    paragraph 4: the pair (T_C, S(C|0)) is stored at first prefill and reuse
 *    composes T_C2*S(C1) + S(C2); the families that need T_C are RetNet,
 *    Mamba2, GLA, DeltaNet, GDN, KDA; conv variants get a "convolution state
 *    warm-up" patch.
 *  - "Hypic: Position-Independent KV Caching ..." (podcast companion page),
 *    sections "The transition operator: compose, don't add" and "Family
 *    comparison: scalar -> diagonal -> dense", plus its reference 7 (Gated
 *    Delta Networks) for the dense transition alpha*(I - beta k k^T).
 *
 * The pages print no equations.  The reading used here (S is d_k x d_v and is
 * left-multiplied by the transition, the current token's write is not decayed,
 * diagonal gates act on the key dimension) is
 *
 *      S_t = A_t S_{t-1} + beta_t k_t v_t^T,    S_0 = 0
 *      scalar    A_t = alpha_t I
 *      diagonal  A_t = diag(alpha_t)           (alpha_t in (0,1)^{d_k})
 *      GDN       A_t = alpha_t (I - beta_t k_t k_t^T)
 *      KDA       A_t = (I - beta_t k_t k_t^T) diag(alpha_t)   (alpha_t in (0,1)^{d_k})
 *      T_C = A_n ... A_1,   S(C|0) = S_n,   so  S_n = T_C S_0 + S(C|0).
 *
 * A record is kept in the exactly factored form T_C = e^{ell} P with
 * ell = sum_t log alpha_t (per key channel for the diagonal family) and
 * P = prod_{t=n..1} (I - beta_t k_t k_t^T) (GDN only; P = I otherwise).
 * KDA's per-channel gates do not commute with the projections, so its record
 * holds T_C itself: ell = 0, P = T_C.
 * beta = NULL means beta_t = 1.
 *
 * Everything is computed token by token in fp64, exactly as the recurrence
 * reads; no chunking, blocking or reordering.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_SCALAR = 0, ORACLE_DIAGONAL = 1, ORACLE_GDN = 2, ORACLE_KDA = 3 };

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * One head of one segment, token by token.
 *   k[t*k_ts + i], v[t*v_ts + j], beta[t*b_ts] (or NULL), la[t*la_ts (+ i)]
 * Writes ell (1 value, or d_k for the diagonal family), P (d_k*d_k, GDN and
 * KDA, may be NULL) and S (d_k*d_v).  S0 (d_k*d_v) is the start state, NULL = 0.
 * With q (q[t*q_ts + i]) and o given, also the in-segment output of every token
 * from the state right after that token's update (the readout of the recurrence
 * that the chunked prefill forward computes):
 *      o[t*o_ts + j] = sum_i S_t[i][j] q_t[i]      (o_t = S_t^T q_t)
 * work must hold d_k + d_v doubles.
 */
static void recur_head(int family, int64_t n, int dk, int dv,
                       const double *k, int64_t k_ts,
                       const double *v, int64_t v_ts,
                       const double *beta, int64_t b_ts,
                       const double *la, int64_t la_ts,
                       const double *S0,
                       double *ell, double *P, double *S, double *work,
                       const double *q, int64_t q_ts, double *o, int64_t o_ts)
{
    const int n_ell = family == ORACLE_DIAGONAL ? dk : 1;
    for (int i = 0; i < n_ell; ++i) ell[i] = 0.0;
    if (P) {
        for (int i = 0; i < dk * dk; ++i) P[i] = 0.0;
        for (int i = 0; i < dk; ++i) P[i * dk + i] = 1.0;
    }
    if (S0) memcpy(S, S0, sizeof(double) * (size_t)dk * dv);
    else    memset(S, 0, sizeof(double) * (size_t)dk * dv);

    double *u = work;          /* k^T P  (d_k) */
    double *w = work + dk;     /* k^T S  (d_v) */

    for (int64_t t = 0; t < n; ++t) {
        const double *kt = k + t * k_ts;
        const double *vt = v + t * v_ts;
        const double b = beta ? beta[t * b_ts] : 1.0;

        if (family == ORACLE_GDN) {
            const double lat = la[t * la_ts];
            const double a = exp(lat);
            if (P) {
                /* P <- (I - b k k^T) P */
                for (int j = 0; j < dk; ++j) u[j] = 0.0;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dk; ++j) u[j] += kt[i] * P[i * dk + j];
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dk; ++j) P[i * dk + j] -= b * kt[i] * u[j];
            }
            /* S <- a (I - b k k^T) S + b k v^T */
            for (int j = 0; j < dv; ++j) w[j] = 0.0;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) w[j] += kt[i] * S[i * dv + j];
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    S[i * dv + j] = a * (S[i * dv + j] - b * kt[i] * w[j]) + b * kt[i] * vt[j];
            ell[0] += lat;
        } else if (family == ORACLE_KDA) {
            /* X <- (I - b k k^T) diag(a) X for X = P and X = S, then S += b k v^T */
            const double *lat = la + t * la_ts;
            if (P) {
                for (int i = 0; i < dk; ++i) {
                    const double a = exp(lat[i]);
                    for (int j = 0; j < dk; ++j) P[i * dk + j] *= a;
                }
                for (int j = 0; j < dk; ++j) u[j] = 0.0;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dk; ++j) u[j] += kt[i] * P[i * dk + j];
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dk; ++j) P[i * dk + j] -= b * kt[i] * u[j];
            }
            for (int i = 0; i < dk; ++i) {
                const double a = exp(lat[i]);
                for (int j = 0; j < dv; ++j) S[i * dv + j] *= a;
            }
            for (int j = 0; j < dv; ++j) w[j] = 0.0;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) w[j] += kt[i] * S[i * dv + j];
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) S[i * dv + j] += b * kt[i] * (vt[j] - w[j]);
        } else if (family == ORACLE_SCALAR) {
            const double lat = la[t * la_ts];
            const double a = exp(lat);
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    S[i * dv + j] = a * S[i * dv + j] + b * kt[i] * vt[j];
            ell[0] += lat;
        } else { /* diagonal: one gate per key channel */
            const double *lat = la + t * la_ts;
            for (int i = 0; i < dk; ++i) {
                const double a = exp(lat[i]);
                for (int j = 0; j < dv; ++j)
                    S[i * dv + j] = a * S[i * dv + j] + b * kt[i] * vt[j];
                ell[i] += lat[i];
            }
        }
        if (q && o) {
            const double *qt = q + t * q_ts;
            double *ot = o + t * o_ts;
            for (int j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) ot[j] += S[i * dv + j] * qt[i];
        }
    }
}

/*
 * Records of a packed stream of segments, every head.
 *   k [N][H][d_k], v [N][H][d_v], beta [N][H] (NULL = 1),
 *   log_alpha [N][H] (scalar, GDN) or [N][H][d_k] (diagonal).
 *   seg_offsets[num_segments+1]: segment s is tokens [off[s], off[s+1]).
 *   init_S [num_segments][H][d_k][d_v] start states, NULL = 0.
 * Outputs: ell [segs][H] or [segs][H][d_k]; P [segs][H][d_k][d_k] (GDN, may be
 * NULL); S [segs][H][d_k][d_v].
 * Returns 0, or -1 on a bad argument.
 */
int oracle_forward(int family, int H, int dk, int dv,
                   int num_segments, const int64_t *seg_offsets,
                   const double *k, const double *v, const double *q,
                   const double *beta, const double *log_alpha,
                   const double *init_S,
                   double *ell, double *P, double *S, double *o);

int oracle_build_segments(int family, int H, int dk, int dv,
                          int num_segments, const int64_t *seg_offsets,
                          const double *k, const double *v,
                          const double *beta, const double *log_alpha,
                          const double *init_S,
                          double *ell, double *P, double *S)
{
    return oracle_forward(family, H, dk, dv, num_segments, seg_offsets, k, v, NULL, beta, log_alpha, init_S,
                          ell, P, S, NULL);
}

/*
 * oracle_build_segments plus the in-segment outputs: with q [N][H][d_k] and
 * o [N][H][d_v], o[t][h] = S_t^T q_t for every token t of every segment, S_t
 * being the head's state right after token t in a recurrence that starts at the
 * segment's first token from init_S (or 0).  q = o = NULL: records only.
 */
int oracle_forward(int family, int H, int dk, int dv,
                   int num_segments, const int64_t *seg_offsets,
                   const double *k, const double *v, const double *q,
                   const double *beta, const double *log_alpha,
                   const double *init_S,
                   double *ell, double *P, double *S, double *o)
{
    if ((q == NULL) != (o == NULL)) return -1;
    if (family < 0 || family > 3 || H <= 0 || dk <= 0 || dv <= 0 || num_segments < 0) return -1;
    if (!seg_offsets || !k || !v || !log_alpha || !ell || !S) return -1;
    for (int s = 0; s < num_segments; ++s)
        if (seg_offsets[s + 1] < seg_offsets[s] || seg_offsets[s] < 0) return -1;

    const int n_ell = family == ORACLE_DIAGONAL ? dk : 1;
    const int per_channel = family == ORACLE_DIAGONAL || family == ORACLE_KDA;
    const int64_t la_ts = per_channel ? (int64_t)H * dk : H;
    const int64_t units = (int64_t)num_segments * H;

#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * (size_t)(dk + dv));
#pragma omp for schedule(dynamic, 1)
        for (int64_t unit = 0; unit < units; ++unit) {
            const int s = (int)(unit / H), h = (int)(unit % H);
            const int64_t t0 = seg_offsets[s];
            const int64_t n = seg_offsets[s + 1] - t0;
            const size_t rec = (size_t)s * H + h;
            const double *la = per_channel ? log_alpha + t0 * la_ts + (int64_t)h * dk
                                           : log_alpha + t0 * la_ts + h;
            recur_head(family, n, dk, dv,
                       k + (t0 * H + h) * dk, (int64_t)H * dk,
                       v + (t0 * H + h) * dv, (int64_t)H * dv,
                       beta ? beta + t0 * H + h : NULL, H,
                       la, la_ts,
                       init_S ? init_S + rec * dk * dv : NULL,
                       ell + rec * n_ell,
                       ((family == ORACLE_GDN || family == ORACLE_KDA) && P) ? P + rec * dk * dk : NULL,
                       S + rec * dk * dv, work,
                       q ? q + (t0 * H + h) * dk : NULL, (int64_t)H * dk,
                       o ? o + (t0 * H + h) * dv : NULL, (int64_t)H * dv);
        }
        free(work);
    }
    return 0;
}

/*
 * Composition of pool records in prompt order, per (request, head):
 *      S <- T_i S + S_i = e^{ell_i} (P_i S) + S_i        (GDN; KDA with ell_i = 0)
 *      S <- e^{ell_i} S + S_i                             (scalar)
 *      S <- diag(e^{ell_i}) S + S_i                       (diagonal)
 * The composed operator is accumulated too: ell <- ell + ell_i and, for GDN
 * when out_P is given, P <- P_i P.
 *   pool_ell [slots][H] (or [slots][H][d_k]), pool_P [slots][H][d_k][d_k]
 *   (GDN), pool_S [slots][H][d_k][d_v];
 *   chain r is chain_slots[chain_offsets[r] .. chain_offsets[r+1]).
 *   init_S [R][H][d_k][d_v] or NULL (zero start).
 * Outputs out_S [R][H][d_k][d_v]; out_ell [R][H] (or [R][H][d_k]) and out_P
 * [R][H][d_k][d_k] when non-NULL.
 * Returns 0, or -1 on a bad argument (including a slot out of range).
 */
int oracle_compose(int family, int H, int dk, int dv, int64_t num_slots,
                   const double *pool_ell, const double *pool_P, const double *pool_S,
                   int R, const int64_t *chain_offsets, const int32_t *chain_slots,
                   const double *init_S,
                   double *out_S, double *out_ell, double *out_P)
{
    if (family < 0 || family > 3 || H <= 0 || dk <= 0 || dv <= 0 || R < 0) return -1;
    if (!pool_ell || !pool_S || !chain_offsets || !out_S) return -1;
    const int dense = family == ORACLE_GDN || family == ORACLE_KDA;   /* records with P */
    if (dense && !pool_P) return -1;
    for (int r = 0; r < R; ++r) {
        if (chain_offsets[r + 1] < chain_offsets[r] || chain_offsets[r] < 0) return -1;
        for (int64_t c = chain_offsets[r]; c < chain_offsets[r + 1]; ++c)
            if (chain_slots[c] < 0 || chain_slots[c] >= num_slots) return -1;
    }
    const int n_ell = family == ORACLE_DIAGONAL ? dk : 1;
    const int64_t units = (int64_t)R * H;
    int status = 0;

#pragma omp parallel
    {
        double *tmp = (double *)malloc(sizeof(double) * (size_t)dk * (dk > dv ? dk : dv));
        double *Pacc = (double *)malloc(sizeof(double) * (size_t)dk * dk);
        double *ellacc = (double *)malloc(sizeof(double) * (size_t)n_ell);
#pragma omp for schedule(dynamic, 1)
        for (int64_t unit = 0; unit < units; ++unit) {
            const int r = (int)(unit / H), h = (int)(unit % H);
            const size_t orec = (size_t)r * H + h;
            double *S = out_S + orec * dk * dv;
            if (init_S) memcpy(S, init_S + orec * dk * dv, sizeof(double) * (size_t)dk * dv);
            else memset(S, 0, sizeof(double) * (size_t)dk * dv);
            for (int i = 0; i < n_ell; ++i) ellacc[i] = 0.0;
            for (int i = 0; i < dk * dk; ++i) Pacc[i] = 0.0;
            for (int i = 0; i < dk; ++i) Pacc[i * dk + i] = 1.0;

            for (int64_t c = chain_offsets[r]; c < chain_offsets[r + 1]; ++c) {
                const size_t rec = (size_t)chain_slots[c] * H + h;
                const double *ell_i = pool_ell + rec * n_ell;
                const double *S_i = pool_S + rec * dk * dv;
                if (dense) {
                    const double *P_i = pool_P + rec * dk * dk;
                    const double sc = exp(ell_i[0]);
                    /* tmp = P_i S */
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dv; ++j) {
                            double acc = 0.0;
                            for (int m = 0; m < dk; ++m) acc += P_i[i * dk + m] * S[m * dv + j];
                            tmp[i * dv + j] = acc;
                        }
                    for (int i = 0; i < dk * dv; ++i) S[i] = sc * tmp[i] + S_i[i];
                    if (out_P) {
                        /* Pacc <- P_i Pacc */
                        for (int i = 0; i < dk; ++i)
                            for (int j = 0; j < dk; ++j) {
                                double acc = 0.0;
                                for (int m = 0; m < dk; ++m) acc += P_i[i * dk + m] * Pacc[m * dk + j];
                                tmp[i * dk + j] = acc;
                            }
                        memcpy(Pacc, tmp, sizeof(double) * (size_t)dk * dk);
                    }
                    ellacc[0] += ell_i[0];
                } else if (family == ORACLE_SCALAR) {
                    const double sc = exp(ell_i[0]);
                    for (int i = 0; i < dk * dv; ++i) S[i] = sc * S[i] + S_i[i];
                    ellacc[0] += ell_i[0];
                } else {
                    for (int i = 0; i < dk; ++i) {
                        const double sc = exp(ell_i[i]);
                        for (int j = 0; j < dv; ++j) S[i * dv + j] = sc * S[i * dv + j] + S_i[i * dv + j];
                        ellacc[i] += ell_i[i];
                    }
                }
            }
            if (out_ell) memcpy(out_ell + orec * n_ell, ellacc, sizeof(double) * (size_t)n_ell);
            if (out_P && dense)
                memcpy(out_P + orec * dk * dk, Pacc, sizeof(double) * (size_t)dk * dk);
        }
        free(tmp);
        free(Pacc);
        free(ellacc);
    }
    return status;
}

/*
 * Causal depthwise convolution over one raw stream, zero history:
 *      y[t][c] = act( bias[c] + sum_{j=0..K-1} w[c][j] * x[t-(K-1)+j][c] ),  x[<0] = 0
 * w[c][K-1] multiplies the current token.  act: 0 identity, 1 SiLU.
 * x [n][C], w [C][K], bias [C] or NULL, y [n][C].
 */
int oracle_causal_conv(int64_t n, int C, int K, const double *x, const double *w,
                       const double *bias, int act, double *y)
{
    if (n < 0 || C <= 0 || K <= 0 || (act != 0 && act != 1)) return -1;
    if ((n > 0 && (!x || !y)) || !w) return -1;
#pragma omp parallel for schedule(static)
    for (int c = 0; c < C; ++c) {
        for (int64_t t = 0; t < n; ++t) {
            double acc = bias ? bias[c] : 0.0;
            for (int j = 0; j < K; ++j) {
                const int64_t src = t - (K - 1) + j;
                if (src >= 0) acc += w[(int64_t)c * K + j] * x[src * C + c];
            }
            y[t * C + c] = act == 1 ? acc / (1.0 + exp(-acc)) : acc;
        }
    }
    return 0;
}
