// Segment-record build for the KDA family (besthub article "Cut First-Token
// Latency by 3.25x ...", paragraph 4, lists KDA among the families whose reuse
// needs the transition operator):
//     A_t = (I - beta_t k_t k_t^T) diag(alpha_t),   S_t = A_t S_{t-1} + beta_t k_t v_t^T,
// with one gate per key channel.  The gates do not commute with the
// projections, so T_C does not factor into a scalar times a gate-free product:
// the record holds T_C itself (P = T_C, ell = 0), and the dense compose applies
// it as it applies a GDN record.
//
// Token-serial fp32 kernel, for the shapes other than d_k = d_v = 128 (those take
// the chunked kernel on the matrix cores).  Workgroup q of a (segment, head) keeps
// 64 of the d_k + d_v columns of [T | S]; four consecutive threads share a column,
// each with d_k / 4 of its rows in registers, so a token is, per thread, a row
// scale, a partial dot product with k (summed over the four with two shuffles)
// and a rank-1 correction:
//     x <- diag(alpha_t) x;   u = k_t^T x;   x <- x + beta_t k_t (v_t[j] - u)
// (v_t[j] only in the S columns).  Each 32-token chunk of k, e^{log alpha}, v
// and beta is staged in LDS first; the token loop reads it with broadcast loads.
#include "hypic_internal.h"

namespace hypic {
namespace {

struct KdaArgs {
    BuildArgs b;
    int32_t nq;          // workgroups per (segment, head)
};

constexpr int NT = 256;
constexpr int CH = 32;
constexpr int DM = 128;
constexpr int COLS = NT / 4;           // columns per workgroup

struct KdaSmem {
    float k[CH][DM];
    float a[CH][DM];     // e^{log alpha}
    float v[CH][COLS];   // this workgroup's S columns of v
    float b[CH];
    int64_t t0, n;
    int32_t slot, state;
};

template <typename XT, int DK>
__global__ __launch_bounds__(NT) void kda_build_kernel(KdaArgs ka) {
    const BuildArgs &a = ka.b;
    constexpr int R = DK / 4;            // rows per thread
    __shared__ KdaSmem sm;
    const int th = threadIdx.x;
    const int nq = ka.nq;
    const int q = blockIdx.x % nq;
    const int head = (blockIdx.x / nq) % a.H;
    const int seg = blockIdx.x / (nq * a.H);
    const int dv = a.dv;
    const int col = q * COLS + (th >> 2);             // column of [T | S]
    const int r0 = (th & 3) * R;                      // this thread's first row
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

    const bool isP = col < DK, isS = col >= DK && col < DK + dv;
    const int scol0 = q * COLS - DK;                  // first S column of this workgroup (if any)
    float x[R];
#pragma unroll
    for (int i = 0; i < R; ++i) x[i] = (isP && r0 + i == col) ? 1.0f : 0.0f;

    // The next chunk's k, log alpha, v and beta are fetched into registers (a fixed
    // number per thread, all issued together) while the current chunk is processed;
    // entries past the segment read its last token and are not used.
    constexpr int NKE = CH * DK / NT, NVE = CH * COLS / NT;
    float fk[NKE], fa[NKE], fv[NVE], fb = 0.f;
    auto fetch = [&](int64_t c0) {
        const int cl = n - c0 < CH ? (int)(n - c0) : CH;
#pragma unroll
        for (int u = 0; u < NKE; ++u) {
            const int e = th + NT * u, t = e / DK, i = e % DK;
            const int64_t tok = t0 + c0 + (t < cl ? t : cl - 1);
            fk[u] = load_f32(kp + tok * a.k_st + head * a.k_sh + i);
            fa[u] = a.log_alpha ? a.log_alpha[tok * a.la_st + head * a.la_sh + i] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < NVE; ++u) {
            const int e = th + NT * u, t = e / COLS, j = e % COLS;
            const int64_t tok = t0 + c0 + (t < cl ? t : cl - 1);
            const int sj = scol0 + j;
            fv[u] = (sj >= 0 && sj < dv) ? load_f32(vp + tok * a.v_st + head * a.v_sh + sj) : 0.0f;
        }
        if (th < CH) {
            const int64_t tok = t0 + c0 + (th < cl ? th : cl - 1);
            fb = a.beta ? a.beta[tok * a.b_st + head * a.b_sh] : 1.0f;
        }
    };
    if (n > 0) fetch(0);
    for (int64_t c0 = 0; c0 < n; c0 += CH) {
        const int cl = n - c0 < CH ? (int)(n - c0) : CH;
        __syncthreads();                      // the previous chunk's tiles are read
#pragma unroll
        for (int u = 0; u < NKE; ++u) {
            const int e = th + NT * u, t = e / DK, i = e % DK;
            sm.k[t][i] = fk[u];
            sm.a[t][i] = expf(fa[u]);
        }
#pragma unroll
        for (int u = 0; u < NVE; ++u) {
            const int e = th + NT * u;
            sm.v[e / COLS][e % COLS] = fv[u];
        }
        if (th < CH) sm.b[th] = fb;
        __syncthreads();
        if (c0 + CH < n) fetch(c0 + CH);
        for (int t = 0; t < cl; ++t) {
            float u0 = 0.f, u1 = 0.f;
#pragma unroll
            for (int i = 0; i < R; i += 4) {
                const float4 al = *reinterpret_cast<const float4 *>(&sm.a[t][r0 + i]);
                const float4 kk = *reinterpret_cast<const float4 *>(&sm.k[t][r0 + i]);
                x[i] *= al.x; x[i + 1] *= al.y; x[i + 2] *= al.z; x[i + 3] *= al.w;
                u0 += kk.x * x[i] + kk.z * x[i + 2];
                u1 += kk.y * x[i + 1] + kk.w * x[i + 3];
            }
            float u = u0 + u1;
            u += __shfl_xor(u, 1);
            u += __shfl_xor(u, 2);              // the column's four row quarters
            const float cf = sm.b[t] * ((isS ? sm.v[t][th >> 2] : 0.0f) - u);
#pragma unroll
            for (int i = 0; i < R; i += 4) {
                const float4 kk = *reinterpret_cast<const float4 *>(&sm.k[t][r0 + i]);
                x[i] += kk.x * cf; x[i + 1] += kk.y * cf; x[i + 2] += kk.z * cf; x[i + 3] += kk.w * cf;
            }
        }
    }
    const float nanv = __int_as_float(0x7fc00000);
    const bool bad = state == 2;
    if (isP) {
        float *P = a.pool_P + rec * DK * DK + col;
#pragma unroll
        for (int i = 0; i < R; ++i) P[(int64_t)(r0 + i) * DK] = bad ? nanv : x[i];
    } else if (isS) {
        float *S = a.pool_S + rec * DK * dv + (col - DK);
#pragma unroll
        for (int i = 0; i < R; ++i) S[(int64_t)(r0 + i) * dv] = bad ? nanv : x[i];
    }
    if (th == 0 && q == 0) a.pool_ell[rec] = bad ? nanv : 0.0f;
}

}  // namespace

hipError_t launch_build_kda(const BuildArgs &b, hipStream_t stream) {
    if (b.num_segments <= 0) return hipSuccess;
    if (b.dk == 128 && b.dv == 128) return launch_build_kda_mfma(b, stream);
    KdaArgs a;
    a.b = b;
    a.nq = (b.dk + b.dv + COLS - 1) / COLS;
    const dim3 grid((unsigned)((int64_t)b.num_segments * b.H * a.nq));
#define HYPIC_KDA(XT_)                                                                      \
    do {                                                                                    \
        if (b.dk == 64) hipLaunchKernelGGL((kda_build_kernel<XT_, 64>), grid, dim3(NT), 0, stream, a); \
        else hipLaunchKernelGGL((kda_build_kernel<XT_, 128>), grid, dim3(NT), 0, stream, a);           \
    } while (0)
    if (b.kv_dtype == HYPIC_BF16) HYPIC_KDA(uint16_t);
    else HYPIC_KDA(float);
#undef HYPIC_KDA
    return hipGetLastError();
}

}  // namespace hypic
