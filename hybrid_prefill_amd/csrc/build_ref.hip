// Segment-record build, fp32 LDS-tiled kernel for every family, d_k, d_v and
// k/v dtype.  This is the exact-arithmetic path (fp32 products, fp64 ell):
// it serves fp32 inputs and any shape the MFMA kernels do not take.
//
// What it computes (besthub article "Cut First-Token Latency by 3.25x ...",
// paragraph 4; agihunt summary, "Core Approach"): for every segment and head
// the record (ell, P, S) with T_C = e^ell P, S = S(C|0) of
//     S_t = A_t S_{t-1} + beta_t k_t v_t^T.
//
// Chunked form.  Tokens are taken 64 at a time (a "chunk").  In a chunk with
// inclusive cumulative log-decay g_t (g over the chunk's tokens, G = g_64),
// keys K (64 x d_k), values V, write gates beta, the GDN step is the WY/UT
// form of the delta rule (Gated Delta Networks, podcast companion page,
// reference 7):
//   A0[t][s]   = beta_t k_t.k_s            (s < t)    ungated, for P
//   A[t][s]    = A0[t][s] e^{g_t - g_s}    (s < t)    gated, for S
//   P-columns:  y = (I + A0)^{-1} (beta . (K P_col));       P_col <- P_col - K^T y
//   S-columns:  y = (I + A )^{-1} (beta . (V_col - e^{g} . (K S_col)));
//               S_col <- e^{G} S_col + (e^{G-g} . K)^T y
// and ell <- ell + G.  The P update uses the ungated system, so P never
// meets a decay factor and cannot overflow however strong the decay.
// Scalar / diagonal families have no P and no solve:
//   S <- e^{G} S + (e^{G-g} . K)^T (beta . V)     (G, g per key channel for diagonal).
// A chunk shorter than 64 tokens is padded with k = v = 0, beta = 0,
// log alpha = 0, which are exact identity transitions.
//
// Work split.  One workgroup per (segment, head, 64-column slab of [P | S]);
// the slab lives in LDS for the whole segment, the per-chunk Gram/solve work
// is repeated per slab.
#include "hypic_internal.h"

namespace hypic {
namespace {

constexpr int CH = 64;    // tokens per chunk
constexpr int NSL = 64;   // state columns per workgroup
constexpr int NT = 256;   // threads per workgroup

template <int FAM, int DK, int DV, typename KVT>
__global__ __launch_bounds__(NT) void build_ref_kernel(BuildArgs a) {
    constexpr int PSL = (FAM == HYPIC_GDN) ? DK / NSL : 0;
    constexpr int SSL = DV / NSL;
    constexpr int NSLAB = PSL + SSL;

    __shared__ float Ks[CH][DK + 1];     // keys of the chunk (scaled in place for the S update)
    __shared__ float St[DK][NSL + 1];    // the state slab
    __shared__ float Ys[CH][NSL + 1];    // Z, right-hand side, solution / beta.V
    __shared__ float Am[FAM == HYPIC_GDN ? CH : 1][CH + 1];
    __shared__ float gs[CH], bs[CH], las[CH];
    __shared__ float Gd[DK];             // per-channel chunk decay (diagonal)
    __shared__ float Gs;
    __shared__ int64_t sh_t0, sh_n;
    __shared__ int32_t sh_slot, sh_state;

    const int tid = threadIdx.x;
    const int slab = blockIdx.x % NSLAB;
    const int unit = blockIdx.x / NSLAB;
    const int h = unit % a.H;
    const int seg = unit / a.H;
    const bool isP = slab < PSL;
    const int c0 = (isP ? slab : slab - PSL) * NSL;

    if (tid == 0) {
        const int64_t o0 = a.seg_offsets[seg], o1 = a.seg_offsets[seg + 1];
        const int32_t slot = a.dst_slots[seg];
        int st = 0;
        if (slot < 0 || slot >= a.num_slots) st = 1;
        else if (o0 < 0 || o1 < o0 || o1 > a.num_tokens) st = 2;
        if (st == 1 && slab == 0) raise_flag(a.err_flag, HYPIC_EFLAG_SLOT_OUT_OF_RANGE);
        if (st == 2 && slab == 0) raise_flag(a.err_flag, HYPIC_EFLAG_BAD_OFFSETS);
        sh_t0 = o0; sh_n = o1 - o0; sh_slot = slot; sh_state = st;
    }
    __syncthreads();
    const int state = sh_state;
    if (state == 1) return;
    const int64_t t0 = sh_t0;
    const int64_t n = state == 2 ? 0 : sh_n;
    const int64_t slot = sh_slot;

    // thread tiles: (tt, cc) over 64x64 outputs with 4x4 elements, interleaved by 16
    const int tr = tid / 16, tc = tid % 16;

    // state slab init: P = I, S = 0
    for (int e = tid; e < DK * NSL; e += NT) {
        const int i = e / NSL, c = e % NSL;
        St[i][c] = (isP && i == c0 + c) ? 1.0f : 0.0f;
    }
    double ell = 0.0;           // thread 0 (scalar, GDN) / thread i < DK (diagonal)

    const KVT *kp = static_cast<const KVT *>(a.k);
    const KVT *vp = static_cast<const KVT *>(a.v);

    for (int64_t base = 0; base < n; base += CH) {
        const int cl = (int)((n - base) < CH ? (n - base) : CH);
        const int64_t tb = t0 + base;
        __syncthreads();   // previous chunk fully consumed
        // ---- load keys, gates
        for (int e = tid; e < CH * DK; e += NT) {
            const int t = e / DK, i = e % DK;
            Ks[t][i] = t < cl ? load_f32(kp + (tb + t) * a.k_st + h * a.k_sh + i) : 0.0f;
        }
        if (tid < CH) {
            const int t = tid;
            bs[t] = t < cl ? (a.beta ? a.beta[(tb + t) * a.b_st + h * a.b_sh] : 1.0f) : 0.0f;
            if (FAM != HYPIC_DIAGONAL)
                las[t] = (t < cl && a.log_alpha) ? a.log_alpha[(tb + t) * a.la_st + h * a.la_sh] : 0.0f;
        }
        __syncthreads();
        // ---- cumulative decay
        if (FAM != HYPIC_DIAGONAL) {
            if (tid == 0) {
                double acc = 0.0;
                for (int t = 0; t < CH; ++t) { acc += (double)las[t]; gs[t] = (float)acc; }
                Gs = (float)acc;
                ell += acc;
            }
        } else {
            if (tid < DK) {
                const int i = tid;
                float gl[CH];
                double acc = 0.0;
#pragma unroll
                for (int t = 0; t < CH; ++t) {
                    const float x = (t < cl && a.log_alpha) ? a.log_alpha[(tb + t) * a.la_st + h * a.la_sh + i] : 0.0f;
                    acc += (double)x;
                    gl[t] = (float)acc;
                }
                const float G = (float)acc;
                ell += acc;
                Gd[i] = G;
#pragma unroll
                for (int t = 0; t < CH; ++t) Ks[t][i] *= __expf(G - gl[t]);
            }
        }
        __syncthreads();

        if (FAM == HYPIC_GDN) {
            // ---- Gram (gated for S slabs, ungated for P slabs) and Z = K * St
            float gacc[4][4], zacc[4][4];
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q) { gacc[p][q] = 0.f; zacc[p][q] = 0.f; }
            for (int i = 0; i < DK; ++i) {
                float kr[4], ks[4], sv[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) { kr[p] = Ks[tr + 16 * p][i]; ks[p] = Ks[tc + 16 * p][i]; sv[p] = St[i][tc + 16 * p]; }
#pragma unroll
                for (int p = 0; p < 4; ++p)
#pragma unroll
                    for (int q = 0; q < 4; ++q) { gacc[p][q] += kr[p] * ks[q]; zacc[p][q] += kr[p] * sv[q]; }
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int t = tr + 16 * p;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int s = tc + 16 * q;
                    float am = 0.0f;
                    if (s < t) am = bs[t] * gacc[p][q] * (isP ? 1.0f : __expf(gs[t] - gs[s]));
                    Am[t][s] = am;
                    const int c = tc + 16 * q;
                    float r;
                    if (isP) {
                        r = bs[t] * zacc[p][q];
                    } else {
                        const float vv = t < cl ? load_f32(vp + (tb + t) * a.v_st + h * a.v_sh + c0 + c) : 0.0f;
                        r = bs[t] * (vv - __expf(gs[t]) * zacc[p][q]);
                    }
                    Ys[t][c] = r;
                }
            }
            __syncthreads();
            // ---- forward substitution (I + Am) y = r, one column per thread of wave 0;
            //      the other waves turn K into K_hat = e^{G-g} K meanwhile (S slabs)
            if (tid < NSL) {
                const int c = tid;
                for (int t = 1; t < CH; ++t) {
                    float acc = Ys[t][c];
                    for (int s = 0; s < t; ++s) acc -= Am[t][s] * Ys[s][c];
                    Ys[t][c] = acc;
                }
            } else if (!isP) {
                for (int e = tid - NSL; e < CH * DK; e += NT - NSL) {
                    const int t = e / DK, i = e % DK;
                    Ks[t][i] *= __expf(Gs - gs[t]);
                }
            }
        } else {
            // ---- scalar / diagonal: right-hand side beta . V, keys scaled by e^{G-g}
            for (int e = tid; e < CH * NSL; e += NT) {
                const int t = e / NSL, c = e % NSL;
                Ys[t][c] = t < cl ? bs[t] * load_f32(vp + (tb + t) * a.v_st + h * a.v_sh + c0 + c) : 0.0f;
            }
            if (FAM == HYPIC_SCALAR) {
                for (int e = tid; e < CH * DK; e += NT) {
                    const int t = e / DK, i = e % DK;
                    Ks[t][i] *= __expf(Gs - gs[t]);
                }
            }
        }
        __syncthreads();
        // ---- slab update: St = decay . St + sign * Ks^T Ys   (rows i = tr + 16p, p < DK/16)
        {
            constexpr int RP = DK / 16;
            float acc[RP][4];
#pragma unroll
            for (int p = 0; p < RP; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[p][q] = 0.f;
            for (int t = 0; t < CH; ++t) {
                float kv[RP], yv[4];
#pragma unroll
                for (int p = 0; p < RP; ++p) kv[p] = Ks[t][tr + 16 * p];
#pragma unroll
                for (int q = 0; q < 4; ++q) yv[q] = Ys[t][tc + 16 * q];
#pragma unroll
                for (int p = 0; p < RP; ++p)
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[p][q] += kv[p] * yv[q];
            }
#pragma unroll
            for (int p = 0; p < RP; ++p) {
                const int i = tr + 16 * p;
                float dec = 1.0f;
                if (!isP) dec = (FAM == HYPIC_DIAGONAL) ? __expf(Gd[i]) : __expf(Gs);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = tc + 16 * q;
                    St[i][c] = isP ? St[i][c] - acc[p][q] : dec * St[i][c] + acc[p][q];
                }
            }
        }
    }
    __syncthreads();

    // ---- write the record
    const float nanv = __int_as_float(0x7fc00000);
    const bool bad = state == 2;
    const int64_t rec = slot * a.H + h;
    if (isP) {
        float *dst = a.pool_P + rec * DK * DK;
        for (int e = tid; e < DK * NSL; e += NT) {
            const int i = e / NSL, c = e % NSL;
            dst[(int64_t)i * DK + c0 + c] = bad ? nanv : St[i][c];
        }
    } else {
        float *dst = a.pool_S + rec * DK * DV;
        for (int e = tid; e < DK * NSL; e += NT) {
            const int i = e / NSL, c = e % NSL;
            dst[(int64_t)i * DV + c0 + c] = bad ? nanv : St[i][c];
        }
        if (slab == PSL) {
            if (FAM == HYPIC_DIAGONAL) {
                if (tid < DK) a.pool_ell[rec * DK + tid] = bad ? nanv : (float)ell;
            } else if (tid == 0) {
                a.pool_ell[rec] = bad ? nanv : (float)ell;
            }
        }
    }
}

template <int FAM, int DK, int DV>
hipError_t launch_fam(const BuildArgs &a, hipStream_t stream) {
    constexpr int NSLAB = ((FAM == HYPIC_GDN) ? DK / NSL : 0) + DV / NSL;
    const dim3 grid((unsigned)((int64_t)a.num_segments * a.H * NSLAB));
    if (a.kv_dtype == HYPIC_BF16)
        hipLaunchKernelGGL((build_ref_kernel<FAM, DK, DV, uint16_t>), grid, dim3(NT), 0, stream, a);
    else
        hipLaunchKernelGGL((build_ref_kernel<FAM, DK, DV, float>), grid, dim3(NT), 0, stream, a);
    return hipGetLastError();
}

template <int FAM>
hipError_t launch_dims(const BuildArgs &a, hipStream_t stream) {
    if (a.dk == 64 && a.dv == 64) return launch_fam<FAM, 64, 64>(a, stream);
    if (a.dk == 64 && a.dv == 128) return launch_fam<FAM, 64, 128>(a, stream);
    if (a.dk == 128 && a.dv == 64) return launch_fam<FAM, 128, 64>(a, stream);
    return launch_fam<FAM, 128, 128>(a, stream);
}

}  // namespace

hipError_t launch_build_ref(const BuildArgs &a, hipStream_t stream) {
    if (a.family == HYPIC_GDN) return launch_dims<HYPIC_GDN>(a, stream);
    if (a.family == HYPIC_SCALAR) return launch_dims<HYPIC_SCALAR>(a, stream);
    return launch_dims<HYPIC_DIAGONAL>(a, stream);
}

}  // namespace hypic
