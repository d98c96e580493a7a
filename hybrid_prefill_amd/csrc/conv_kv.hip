// Keys and values of chosen tokens of a conv variant, from raw inputs (besthub
// article "Cut First-Token Latency by 3.25x ...", paragraph 4: conv variants need
// a convolution state warm-up so that reused segments stay aligned).
//
// In a conv variant the recurrence does not see the projected inputs x directly:
// a causal depthwise conv of kernel size K runs over time first, then an
// activation, and the keys are L2-normalised per head.  For output token t with
// window rows win[t][0..K-1] of the raw table (row -1 reads as zeros):
//     y[c]      = act( bias[c] + sum_j w[c][j] x[win[t][j]][c] ),   c < C = H (d_k + d_v)
//     k[t][h]   = y[h d_k .. h d_k + d_k) / sqrt(|.|^2 + 1e-6)       (or unnormalised)
//     v[t][h]   = y[H d_k + h d_v .. + d_v)
// and, with src_token, beta and log alpha of output token t gathered from token
// src_token[t] of their streams.  The window rows are the caller's: the tokens
// of a segment after its first K-1 see only the segment itself, the first K-1
// the previous segment's last raw inputs (the warm-up).
//
// One workgroup per output token: the conv is computed channel-parallel into
// LDS (16 bytes of channels per thread and load when the channel count and the
// pointers allow it), then one wave per head reduces the key norm and writes the
// head.
#include "hypic_internal.h"

namespace hypic {
namespace {

constexpr int NT = 256;

template <typename OT>
__device__ __forceinline__ OT to_out(float x) { return (OT)x; }   // bf16: round to nearest even

// 16 bytes of raw inputs: 8 bf16 or 4 fp32 channels, as floats
template <typename XT> struct XV;
template <> struct XV<uint16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void load(const uint16_t *p, float *f) {
        const uint4 r = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct XV<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void load(const float *p, float *f) {
        const float4 r = *reinterpret_cast<const float4 *>(p);
        f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w;
    }
};

template <typename XT, typename OT, bool VEC>
__global__ __launch_bounds__(NT) void conv_kv_kernel(ConvKvArgs a) {
    extern __shared__ float y[];          // [C]
    __shared__ int bad;
    const int t = blockIdx.x;
    const int th = threadIdx.x;
    const int K = a.ksize;
    const int C = a.H * (a.dk + a.dv);
    const XT *x = static_cast<const XT *>(a.x);
    if (th == 0) {
        int b = 0;
        for (int j = 0; j < K; ++j) {
            const int32_t r = a.window[(int64_t)t * K + j];
            if (r < -1 || r >= a.num_rows) b = 1;
        }
        if (a.src_token) {
            const int32_t s = a.src_token[t];
            if (s < 0 || s >= a.num_src_tokens) b = 1;
        }
        if (b) raise_flag(a.err_flag, HYPIC_EFLAG_SLOT_OUT_OF_RANGE);
        bad = b;
    }
    __syncthreads();
    const float nanv = __int_as_float(0x7fc00000);
    OT *ko = static_cast<OT *>(a.k_out) + (int64_t)t * a.H * a.dk;
    OT *vo = static_cast<OT *>(a.v_out) + (int64_t)t * a.H * a.dv;
    if (bad) {
        for (int c = th; c < a.H * a.dk; c += NT) ko[c] = to_out<OT>(nanv);
        for (int c = th; c < a.H * a.dv; c += NT) vo[c] = to_out<OT>(nanv);
        if (a.src_token)
            for (int h = th; h < a.H; h += NT) {
                a.beta_out[(int64_t)t * a.H + h] = nanv;
                a.la_out[(int64_t)t * a.H + h] = nanv;
            }
        return;
    }
    int32_t rows[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) rows[j] = j < K ? a.window[(int64_t)t * K + j] : -1;
    if constexpr (VEC) {
        // kernel size 4: a channel's taps are one 16-byte load
        constexpr int NV = XV<XT>::N;
        const float4 *w4 = reinterpret_cast<const float4 *>(a.weight);
        for (int c0 = NV * th; c0 < C; c0 += NV * NT) {
            float acc[NV];
            float4 wv[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                acc[i] = a.bias ? a.bias[c0 + i] : 0.0f;
                wv[i] = w4[c0 + i];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (rows[j] >= 0) {
                    float xv[NV];
                    XV<XT>::load(x + (int64_t)rows[j] * C + c0, xv);
#pragma unroll
                    for (int i = 0; i < NV; ++i) {
                        const float wj = j == 0 ? wv[i].x : j == 1 ? wv[i].y : j == 2 ? wv[i].z : wv[i].w;
                        acc[i] += wj * xv[i];
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                float v = acc[i];
                if (a.activation == 1) v = v / (1.0f + expf(-v));
                y[c0 + i] = v;
            }
        }
    } else {
        for (int c = th; c < C; c += NT) {
            float acc = a.bias ? a.bias[c] : 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < K && rows[j] >= 0) acc += a.weight[(int64_t)c * K + j] * load_f32(x + (int64_t)rows[j] * C + c);
            if (a.activation == 1) acc = acc / (1.0f + expf(-acc));
            y[c] = acc;
        }
    }
    __syncthreads();
    // keys: wave w takes heads w, w + 4, ...; lane l the channels l, l + 64, ...
    const int w = th >> 6, l = th & 63;
    for (int h = w; h < a.H; h += NT / 64) {
        const float *yh = y + h * a.dk;
        float ss = 0.f;
        for (int i = l; i < a.dk; i += 64) ss += yh[i] * yh[i];
        for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
        const float inv = a.normalize_k ? 1.0f / sqrtf(ss + 1e-6f) : 1.0f;
        for (int i = l; i < a.dk; i += 64) ko[h * a.dk + i] = to_out<OT>(yh[i] * inv);
    }
    for (int c = th; c < a.H * a.dv; c += NT) vo[c] = to_out<OT>(y[a.H * a.dk + c]);
    if (a.src_token) {
        const int64_t s = a.src_token[t];
        for (int h = th; h < a.H; h += NT) {
            a.beta_out[(int64_t)t * a.H + h] = a.beta ? a.beta[s * a.H + h] : 1.0f;
            a.la_out[(int64_t)t * a.H + h] = a.log_alpha ? a.log_alpha[s * a.H + h] : 0.0f;
        }
    }
}

}  // namespace

hipError_t launch_conv_kv(const ConvKvArgs &a, hipStream_t stream) {
    if (a.num_tokens <= 0) return hipSuccess;
    const int C = a.H * (a.dk + a.dv);
    const size_t lds = (size_t)C * sizeof(float);
    const dim3 grid((unsigned)a.num_tokens);
    const bool bf = a.x_dtype == HYPIC_BF16;
    const bool vec = a.ksize == 4 && C % (bf ? 8 : 4) == 0 && ((uintptr_t)a.x & 15) == 0 &&
                     ((uintptr_t)a.weight & 15) == 0;
#define HYPIC_CKV(XT_, OT_)                                                                        \
    do {                                                                                           \
        if (vec) hipLaunchKernelGGL((conv_kv_kernel<XT_, OT_, true>), grid, dim3(NT), lds, stream, a); \
        else hipLaunchKernelGGL((conv_kv_kernel<XT_, OT_, false>), grid, dim3(NT), lds, stream, a);    \
    } while (0)
    if (bf) {
        if (a.out_dtype == HYPIC_BF16) HYPIC_CKV(uint16_t, __bf16);
        else HYPIC_CKV(uint16_t, float);
    } else {
        if (a.out_dtype == HYPIC_BF16) HYPIC_CKV(float, __bf16);
        else HYPIC_CKV(float, float);
    }
#undef HYPIC_CKV
    return hipGetLastError();
}

}  // namespace hypic
