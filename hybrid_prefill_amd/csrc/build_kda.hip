// Segment-record build for the KDA family (besthub article "Cut First-Token
// Latency by 3.25x ...", paragraph 4, lists KDA among the families whose reuse
// needs the transition operator):
//     A_t = (I - beta_t k_t k_t^T) diag(alpha_t),   S_t = A_t S_{t-1} + beta_t k_t v_t^T,
// with one gate per key channel.  The gates do not commute with the
// projections, so T_C does not factor into a scalar times a gate-free product:
// the record holds T_C itself (P = T_C, ell = 0), and the dense compose applies
// it as it applies a GDN record.
//
// Token-serial fp32 kernel (the chunked UT form with per-channel decay inside
// the triangular solve is not built yet): one workgroup per (segment, head),
// thread j owns column j of [T | S] (d_k + d_v <= 256 columns) with its d_k rows
// in registers, so a token is, per thread, a row scale, a dot product with k
// and a rank-1 correction -- no reduction across threads:
//     x <- diag(alpha_t) x;   u = k_t^T x;   x <- x + beta_t k_t (v_t[j] - u)
// (v_t[j] only in the S columns).  Each 64-token chunk of k, e^{log alpha},
// v and beta is staged in LDS first; the token loop reads it with broadcast
// loads.
#include "hypic_internal.h"

namespace hypic {
namespace {

constexpr int NT = 256;
constexpr int CH = 64;
constexpr int DM = 128;

struct KdaSmem {
    float k[CH][DM];
    float a[CH][DM];     // e^{log alpha}
    float v[CH][DM];
    float b[CH];
    int64_t t0, n;
    int32_t slot, state;
};

template <typename XT, int DK>
__global__ __launch_bounds__(NT) void kda_build_kernel(BuildArgs a) {
    __shared__ KdaSmem sm;
    const int th = threadIdx.x;
    const int head = blockIdx.x % a.H;
    const int seg = blockIdx.x / a.H;
    const int dv = a.dv;
    if (th == 0) {
        const int64_t o0 = a.seg_offsets[seg], o1 = a.seg_offsets[seg + 1];
        const int32_t slot = a.dst_slots[seg];
        int st = 0;
        if (slot < 0 || slot >= a.num_slots) st = 1;
        else if (o0 < 0 || o1 < o0 || o1 > a.num_tokens) st = 2;
        if (st == 1) raise_flag(a.err_flag, HYPIC_EFLAG_SLOT_OUT_OF_RANGE);
        if (st == 2) raise_flag(a.err_flag, HYPIC_EFLAG_BAD_OFFSETS);
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

    const bool isP = th < DK, isS = th >= DK && th < DK + dv;
    float x[DK];
#pragma unroll
    for (int i = 0; i < DK; ++i) x[i] = (isP && i == th) ? 1.0f : 0.0f;

    for (int64_t c0 = 0; c0 < n; c0 += CH) {
        const int cl = n - c0 < CH ? (int)(n - c0) : CH;
        __syncthreads();                      // the previous chunk's tiles are read
        for (int e = th; e < cl * DK; e += NT) {
            const int t = e / DK, i = e % DK;
            const int64_t tok = t0 + c0 + t;
            sm.k[t][i] = load_f32(kp + tok * a.k_st + head * a.k_sh + i);
            sm.a[t][i] = a.log_alpha ? expf(a.log_alpha[tok * a.la_st + head * a.la_sh + i]) : 1.0f;
        }
        for (int e = th; e < cl * dv; e += NT) {
            const int t = e / dv, j = e % dv;
            sm.v[t][j] = load_f32(vp + (t0 + c0 + t) * a.v_st + head * a.v_sh + j);
        }
        for (int t = th; t < cl; t += NT) sm.b[t] = a.beta ? a.beta[(t0 + c0 + t) * a.b_st + head * a.b_sh] : 1.0f;
        __syncthreads();
        if (isP || isS) {
            for (int t = 0; t < cl; ++t) {
                float u = 0.f;
#pragma unroll
                for (int i = 0; i < DK; i += 4) {
                    const float4 al = *reinterpret_cast<const float4 *>(&sm.a[t][i]);
                    const float4 kk = *reinterpret_cast<const float4 *>(&sm.k[t][i]);
                    x[i] *= al.x; x[i + 1] *= al.y; x[i + 2] *= al.z; x[i + 3] *= al.w;
                    u += kk.x * x[i] + kk.y * x[i + 1] + kk.z * x[i + 2] + kk.w * x[i + 3];
                }
                const float cf = sm.b[t] * ((isS ? sm.v[t][th - DK] : 0.0f) - u);
#pragma unroll
                for (int i = 0; i < DK; i += 4) {
                    const float4 kk = *reinterpret_cast<const float4 *>(&sm.k[t][i]);
                    x[i] += kk.x * cf; x[i + 1] += kk.y * cf; x[i + 2] += kk.z * cf; x[i + 3] += kk.w * cf;
                }
            }
        }
    }
    const float nanv = __int_as_float(0x7fc00000);
    const bool bad = state == 2;
    if (isP) {
        float *P = a.pool_P + rec * DK * DK + th;
#pragma unroll
        for (int i = 0; i < DK; ++i) P[(int64_t)i * DK] = bad ? nanv : x[i];
    } else if (isS) {
        float *S = a.pool_S + rec * DK * dv + (th - DK);
#pragma unroll
        for (int i = 0; i < DK; ++i) S[(int64_t)i * dv] = bad ? nanv : x[i];
    }
    if (th == 0) a.pool_ell[rec] = bad ? nanv : 0.0f;
}

}  // namespace

hipError_t launch_build_kda(const BuildArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)a.num_segments * a.H));
    if (a.num_segments <= 0) return hipSuccess;
#define HYPIC_KDA(XT_)                                                                      \
    do {                                                                                    \
        if (a.dk == 64) hipLaunchKernelGGL((kda_build_kernel<XT_, 64>), grid, dim3(NT), 0, stream, a); \
        else hipLaunchKernelGGL((kda_build_kernel<XT_, 128>), grid, dim3(NT), 0, stream, a);           \
    } while (0)
    if (a.kv_dtype == HYPIC_BF16) HYPIC_KDA(uint16_t);
    else HYPIC_KDA(float);
#undef HYPIC_KDA
    return hipGetLastError();
}

}  // namespace hypic
