// Chunked segment-record build for the KDA family at d_k = d_v = 128 on the fp32
// matrix cores (besthub article "Cut First-Token Latency by 3.25x ...",
// paragraph 4, lists KDA among the families whose reuse needs the transition
// operator):
//     A_t = (I - beta_t k_t k_t^T) diag(alpha_t),   X_t = A_t X_{t-1} + beta_t k_t [0 | v_t^T],
// on X = [T | S] (d_k rows, d_k + d_v columns, X_0 = [I | 0]); the record is
// (ell = 0, P = T_C, S).
//
// Chunk form (32 tokens, g_t = the chunk's cumulative log alpha up to and
// including token t, per key channel).  Writing each token's correction as
// e_t = beta_t (v_t - k_t^T diag(alpha_t) X_{t-1}) (a row, zero v in the T
// columns), unrolling the recurrence over the chunk gives
//     X_t = diag(e^{g_t}) X_0 + sum_{s<=t} diag(e^{g_t - g_s}) k_s e_s,
//     (I + diag(beta) A) E = diag(beta) (V - K_g X_0),
//     A_ts = sum_i k_t[i] k_s[i] e^{g_t[i] - g_s[i]}  (s < t),  K_g row t = k_t e^{g_t},
// so with T = (I + diag(beta) A)^{-1} (unit lower triangular),
// M = T diag(beta) K_g and U = T diag(beta) V, which do not depend on the state:
//     E = U - M X_0,     X_C = diag(e^{g_C}) X_0 + Khat^T E,   Khat row s = k_s e^{g_C - g_s}.
// The Gram A is formed in three 16 x 16 blocks, each as a product of two
// per-token scaled key tiles whose exponents are split at a reference token:
// the off-diagonal block at the boundary between the halves (both factors
// <= 1), a diagonal block at its eighth token (factors up to the decay over
// seven tokens).  A chunk whose factors would exceed 2^100 (a channel decaying
// by more than e^-69 within seven tokens) is instead applied token by token to
// the state, from the same staged keys, gates and values.
//
// Workgroup (segment, head, q): q = 0 keeps the T columns, q = 1 the S columns;
// wave w keeps 32 of them as four 32 x 32 fp32 accumulator tiles.  Per chunk:
// staging (thread per key channel and token half: prefix of the gates,
// scaled keys into LDS), Gram blocks (waves 0-2, 16x16x4 fp32 MFMA), inversion
// (wave 0, lane per column, forward substitution), M and U (every wave, its 32
// channels of M and its 32 columns of U, 32x32x2 fp32 MFMA), then E and the
// state update on the wave's own columns.
#include "hypic_internal.h"

namespace hypic {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NT = 256;
constexpr int CK = 32;                  // tokens per chunk
constexpr int D = 128;
constexpr int LP = 132;                 // row stride of the [CK][D] tiles (floats)
constexpr int TP = 36;                  // row stride of the [D][CK] and [CK][CK] tiles
constexpr float LOG2E = 1.4426950408889634f;
constexpr float EXP_LIMIT = 100.0f;     // largest base-2 exponent a scaled key may carry

struct KdaMfmaSmem {
    float kg[CK][LP];      // k_t e^{g_t}
    float qd[CK][LP];      // diagonal blocks, query side; then -M.   Serial chunk: raw k
    float kd[CK][LP];      // diagonal blocks, key side.              Serial chunk: e^{log alpha}
    float x1[CK][LP];      // off-diagonal block: key side (rows 0..15), query side (rows 16..31)
    float v[CK][LP];       // v of this workgroup's columns (S workgroup)
    float kht[D][TP];      // Khat^T
    float nm[CK][TP];      // beta_t A_ts for s < t
    float tw[4][CK][TP];   // per wave: T (diagonal blocks)
    float tn[4][CK][TP];   // per wave: -T diag(beta) (upper right block zero)
    float gam[D];          // e^{g_C}
    float b[CK];
    int64_t t0, n;
    int32_t slot, state;
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename XT>
__global__ __launch_bounds__(NT, 1) void kda_chunk_mfma_kernel(BuildArgs a) {
    __shared__ KdaMfmaSmem sm;
    const int th = threadIdx.x, lane = th & 63, w = th >> 6;
    const int q = blockIdx.x & 1;
    const int head = (blockIdx.x >> 1) % a.H;
    const int seg = (blockIdx.x >> 1) / a.H;
    if (th == 0) {
        const int64_t o0 = a.seg_offsets[seg], o1 = a.seg_offsets[seg + 1];
        const int32_t slot = a.dst_slots[seg];
        int st = 0;
        if (slot < 0 || slot >= a.num_slots) st = 1;
        else if (o0 < 0 || o1 < o0 || o1 > a.num_tokens) st = 2;
        if (st == 1 && q == 0) raise_flag(a.err_flag, HYPIC_EFLAG_SLOT_OUT_OF_RANGE);
        if (st == 2 && q == 0) raise_flag(a.err_flag, HYPIC_EFLAG_BAD_OFFSETS);
        sm.t0 = o0; sm.n = o1 - o0; sm.slot = slot; sm.state = st;
    }
    __syncthreads();
    const int state = sm.state;
    if (state == 1) return;
    const int64_t t0 = sm.t0;
    const int64_t n = state == 2 ? 0 : sm.n;
    const int64_t rec = (int64_t)sm.slot * a.H + head;
    const XT *kp = static_cast<const XT *>(a.k);
    const XT *vp = static_cast<const XT *>(a.v);
    const bool isS = q == 1;

    // MFMA role: lane (ln, hh) of wave w keeps column colw, rows 32r + 8(i/4) + 4hh + i%4.
    const int ln = lane & 31, hh = lane >> 5;
    const int colw = 32 * w + ln;
    f32x16 X[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            X[r][i] = (!isS && 32 * r + 8 * (i >> 2) + 4 * hh + (i & 3) == colw) ? 1.0f : 0.0f;

    // Staging role: key channel ch (also the value column), tokens 16hf .. 16hf+15.
    // The next chunk's inputs are fetched into registers while the current one runs.
    // The loads take no branch (a branch joining around a load makes the compiler
    // wait for it there): entries past the segment read its last token, a missing
    // log alpha or beta is read from the keys with stride 0, and the selects that
    // replace them (zero gates and values, unit or zero beta) are applied at use.
    const int ch = th & 127, hf = th >> 7;
    const bool has_la = a.log_alpha != nullptr, has_b = a.beta != nullptr;
    const float *la_p = has_la ? a.log_alpha + head * a.la_sh + ch : static_cast<const float *>(a.k);
    const int64_t la_st = has_la ? a.la_st : 0;
    const float *b_p = has_b ? a.beta + head * a.b_sh : static_cast<const float *>(a.k);
    const int64_t b_st = has_b ? a.b_st : 0;
    const XT *k_p = kp + head * a.k_sh + ch;
    const XT *v_p = vp + head * a.v_sh + ch;
    float rla[CK], rk[16], rv[16], rb;
    auto fetch = [&](int64_t c0) {
        const int cl = n - c0 < CK ? (int)(n - c0) : CK;
        const int64_t base = t0 + c0;
#pragma unroll
        for (int t = 0; t < CK; ++t) rla[t] = la_p[(base + (t < cl ? t : cl - 1)) * la_st];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int t = 16 * hf + u;
            const int64_t tok = base + (t < cl ? t : cl - 1);
            rk[u] = load_f32(k_p + tok * a.k_st);
            rv[u] = load_f32(v_p + tok * a.v_st);
        }
        const int tb_ = th & (CK - 1);
        rb = b_p[(base + (tb_ < cl ? tb_ : cl - 1)) * b_st];
    };
    // The upper right block of every wave's -T diag(beta) stays zero.
    for (int e = th; e < 4 * 16 * 16; e += NT) sm.tn[e >> 8][(e >> 4) & 15][16 + (e & 15)] = 0.0f;
    if (n > 0) fetch(0);

    for (int64_t c0 = 0; c0 < n; c0 += CK) {
        const int cl = n - c0 < CK ? (int)(n - c0) : CK;
        float G[CK];
        {
            float acc = 0.0f;
#pragma unroll
            for (int t = 0; t < CK; ++t) {
                acc += (t < cl && has_la ? rla[t] : 0.0f) * LOG2E;
                G[t] = acc;
            }
        }
        const float Gc = G[CK - 1], Gh = G[15], Gr = hf ? G[23] : G[7];
        // This thread's half of the prefix (a select per token: indexing G by the
        // runtime half would compile to a compare-and-select over all 32 registers).
        float Gs[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) Gs[u] = hf ? G[16 + u] : G[u];
        float emax = -INFINITY;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float g = Gs[u];
            emax = fmaxf(emax, fmaxf(fmaxf(g, Gc - g), fmaxf(g - Gr, Gr - g)));
            emax = fmaxf(emax, hf ? g - Gh : Gh - g);
        }
        // Also the barrier after the previous chunk's last reads of the tiles.
        const bool serial = __syncthreads_or(!(emax <= EXP_LIMIT)) != 0;
        if (!serial) {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int t = 16 * hf + u;
                const float kk = t < cl ? rk[u] : 0.0f, g = Gs[u];
                sm.kg[t][ch] = kk * ex2(g);
                sm.kht[ch][t] = kk * ex2(Gc - g);
                sm.qd[t][ch] = kk * ex2(g - Gr);
                sm.kd[t][ch] = kk * ex2(Gr - g);
                sm.x1[t][ch] = kk * ex2(hf ? g - Gh : Gh - g);
                sm.v[t][ch] = t < cl && isS ? rv[u] : 0.0f;
            }
            if (hf == 0) sm.gam[ch] = ex2(Gc);
        } else {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int t = 16 * hf + u;
                sm.qd[t][ch] = t < cl ? rk[u] : 0.0f;
                const float la_t = hf ? rla[16 + u] : rla[u];
                sm.kd[t][ch] = t < cl && has_la ? ex2(la_t * LOG2E) : 1.0f;
                sm.v[t][ch] = t < cl && isS ? rv[u] : 0.0f;
            }
        }
        if (th < CK) sm.b[th] = th < cl ? (has_b ? rb : 1.0f) : 0.0f;
        fetch(c0 + CK);                     // past the last chunk: the segment's last token again, unused
        __syncthreads();

        if (!serial) {
            // Gram blocks: wave 0 (0,0), wave 1 (1,1), wave 2 (1,0); beta_t A_ts below the diagonal.
            if (w < 3) {
                const float(*Qt)[LP] = w == 2 ? sm.x1 : sm.qd;
                const float(*Kt)[LP] = w == 2 ? sm.x1 : sm.kd;
                const int I = w == 0 ? 0 : 1, J = w == 1 ? 1 : 0;
                const int m = lane & 15, g = lane >> 4;
                f32x4 c0v = {0.f, 0.f, 0.f, 0.f}, c1v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 8; ++s) {      // contraction index 16s + 4g + j
                    const f32x4 qa = *reinterpret_cast<const f32x4 *>(&Qt[16 * I + m][16 * s + 4 * g]);
                    const f32x4 kb = *reinterpret_cast<const f32x4 *>(&Kt[16 * J + m][16 * s + 4 * g]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (s & 1) c1v = mfma16(qa[j], kb[j], c1v);
                        else c0v = mfma16(qa[j], kb[j], c0v);
                    }
                }
                const f32x4 Ab = c0v + c1v;          // rows 16I + 4g + j, column 16J + m
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = 16 * I + 4 * g + j, s = 16 * J + m;
                    sm.nm[t][s] = t > s ? sm.b[t] * Ab[j] : 0.0f;
                }
            }
            __syncthreads();
            // Every wave now works alone until the next chunk (no barrier):
            // (1) W = K_g X_0 - V on its columns (contraction over state rows), which
            //     does not need T, so the scheduler can overlap it with
            // (2) its own copy of T = (I + N)^{-1} (N = diag(beta) A, strictly lower):
            //     the two diagonal 16 x 16 blocks by forward substitution (lane per
            //     column: lanes 0-15 the first block, 16-31 the second, the upper half
            //     of the wave repeating them), then T_10 = -T_11 (N_10 T_00) on the
            //     16x16x4 MFMA; -T diag(beta) goes to the wave's own LDS tile;
            // (3) E = -T diag(beta) W = T diag(beta) (V - K_g X_0);
            // (4) X_C = diag(e^{g_C}) X_0 + Khat^T E.
            f32x16 W0, W1;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                W0[i] = isS ? -sm.v[8 * (i >> 2) + 4 * hh + (i & 3)][colw] : 0.0f;
                W1[i] = 0.0f;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const f32x4 kv = *reinterpret_cast<const f32x4 *>(&sm.kg[ln][32 * r + 8 * s + 4 * hh]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (r & 1) W1 = mfma32(kv[j], X[r][4 * s + j], W1);
                        else W0 = mfma32(kv[j], X[r][4 * s + j], W0);
                    }
                }
            float(*tw)[TP] = sm.tw[w];
            float(*tn)[TP] = sm.tn[w];
            {
                const int c = lane & 15, blk = (lane >> 4) & 1, o = 16 * blk;
                float tc[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) tc[i] = i == c ? 1.0f : 0.0f;
#pragma unroll
                for (int i = 1; i < 16; ++i) {
                    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
                    for (int m4 = 0; m4 < i; m4 += 4) {
                        const f32x4 nv = *reinterpret_cast<const f32x4 *>(&sm.nm[o + i][o + m4]);
                        if (m4 + 0 < i) s0 += nv[0] * tc[m4 + 0];
                        if (m4 + 1 < i) s1 += nv[1] * tc[m4 + 1];
                        if (m4 + 2 < i) s0 += nv[2] * tc[m4 + 2];
                        if (m4 + 3 < i) s1 += nv[3] * tc[m4 + 3];
                    }
                    if (i > c) tc[i] = -(s0 + s1);
                }
                const float bc = sm.b[o + c];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    tw[o + i][o + c] = tc[i];
                    tn[o + i][o + c] = -tc[i] * bc;
                }
            }
            {
                // Y = N_10 T_00, then T_11 Y = -T_10 (contraction index 4g + j at step j).
                const int m = lane & 15, g = lane >> 4;
                const f32x4 na = *reinterpret_cast<const f32x4 *>(&sm.nm[16 + m][4 * g]);
                f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) Y = mfma16(na[j], tw[4 * g + j][m], Y);
                const f32x4 ta = *reinterpret_cast<const f32x4 *>(&tw[16 + m][16 + 4 * g]);
                f32x4 Z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) Z = mfma16(ta[j], Y[j], Z);
                const float bm = sm.b[m];
#pragma unroll
                for (int j = 0; j < 4; ++j) tn[16 + 4 * g + j][m] = Z[j] * bm;
            }
            const f32x16 Wt = W0 + W1;             // rows: the chunk's tokens 8(i/4) + 4hh + i%4
            f32x16 E;
#pragma unroll
            for (int i = 0; i < 16; ++i) E[i] = 0.0f;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const f32x4 ta = *reinterpret_cast<const f32x4 *>(&tn[ln][8 * s + 4 * hh]);
#pragma unroll
                for (int j = 0; j < 4; ++j) E = mfma32(ta[j], Wt[4 * s + j], E);
            }
            // X_C = diag(e^{g_C}) X_0 + Khat^T E.
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const f32x4 gg = *reinterpret_cast<const f32x4 *>(&sm.gam[32 * r + 8 * s + 4 * hh]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) X[r][4 * s + j] *= gg[j];
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const f32x4 kh = *reinterpret_cast<const f32x4 *>(&sm.kht[32 * r + ln][8 * s + 4 * hh]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) X[r] = mfma32(kh[j], E[4 * s + j], X[r]);
                }
            }
        } else {
            // Token by token on the state: the lane pair (ln, 0), (ln, 1) holds the column.
            for (int t = 0; t < cl; ++t) {
                float u = 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int row = 32 * r + 8 * s + 4 * hh;
                        const f32x4 al = *reinterpret_cast<const f32x4 *>(&sm.kd[t][row]);
                        const f32x4 kk = *reinterpret_cast<const f32x4 *>(&sm.qd[t][row]);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            X[r][4 * s + j] *= al[j];
                            u += kk[j] * X[r][4 * s + j];
                        }
                    }
                u += __shfl_xor(u, 32);
                const float cf = sm.b[t] * ((isS ? sm.v[t][colw] : 0.0f) - u);
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const f32x4 kk = *reinterpret_cast<const f32x4 *>(&sm.qd[t][32 * r + 8 * s + 4 * hh]);
#pragma unroll
                        for (int j = 0; j < 4; ++j) X[r][4 * s + j] += kk[j] * cf;
                    }
            }
        }
    }

    const float nanv = __int_as_float(0x7fc00000);
    const bool bad = state == 2;
    float *dst = (isS ? a.pool_S : a.pool_P) + rec * D * D + colw;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            dst[(int64_t)(32 * r + 8 * (i >> 2) + 4 * hh + (i & 3)) * D] = bad ? nanv : X[r][i];
    if (th == 0 && q == 0) a.pool_ell[rec] = bad ? nanv : 0.0f;
}

}  // namespace

hipError_t launch_build_kda_mfma(const BuildArgs &b, hipStream_t stream) {
    if (b.num_segments <= 0) return hipSuccess;
    if (b.dk != D || b.dv != D) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((int64_t)b.num_segments * b.H * 2));
    if (b.kv_dtype == HYPIC_BF16) hipLaunchKernelGGL(kda_chunk_mfma_kernel<uint16_t>, grid, dim3(NT), 0, stream, b);
    else hipLaunchKernelGGL(kda_chunk_mfma_kernel<float>, grid, dim3(NT), 0, stream, b);
    return hipGetLastError();
}

}  // namespace hypic
