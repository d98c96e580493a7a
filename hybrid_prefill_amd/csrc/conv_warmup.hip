// Convolution state warm-up at segment boundaries (besthub article "Cut
// First-Token Latency by 3.25x ...", paragraph 4: conv variants get a
// convolution state warm-up patch so reused segments stay aligned).
//
// A causal depthwise conv of kernel size K precedes the recurrence in conv
// variants.  A segment prefilled alone saw zeros before its first token; on
// reuse its first K-1 outputs are recomputed with the previous segment's last
// K-1 raw inputs as the conv state:
//   x_bar = [tail (K-1 rows); head (K-1 rows)],
//   out[t][c] = act(bias[c] + sum_{j<K} w[c][j] x_bar[t+j][c]),  t < K-1.
// From position K-1 on the window holds only the segment's own tokens, so
// nothing else changes.
//
// Bandwidth-bound.  Main kernel: the boundary is the grid's y index (its table
// indices are wave-uniform scalar loads) and each thread owns 16 bytes of
// channels of every input row (8 bf16 or 4 fp32), so every load is one 16-byte
// access and every output row two or one 16-byte stores, coalesced along C.
// Channel counts or pointers that do not allow that take the one-channel-per-
// thread kernel.
#include "hypic_internal.h"

namespace hypic {
namespace {

constexpr int NT = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename XT, int K>
__global__ __launch_bounds__(NT) void conv_warmup_kernel(ConvArgs a) {
    const int64_t C = a.channels;
    const int64_t total = (int64_t)a.num_boundaries * C;
    const XT *tails = static_cast<const XT *>(a.tails);
    const XT *heads = static_cast<const XT *>(a.heads);
    const float nanv = __int_as_float(0x7fc00000);
    for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < total; e += (int64_t)gridDim.x * NT) {
        const int64_t b = e / C, c = e % C;
        const int64_t ti = a.tail_index ? a.tail_index[b] : b;
        const int64_t hi = a.head_index ? a.head_index[b] : b;
        float *out = a.out + b * (K - 1) * C + c;
        if (ti < 0 || ti >= a.num_tails || hi < 0 || hi >= a.num_heads) {
            if (c == 0) raise_flag(a.err_flag, HYPIC_EFLAG_SLOT_OUT_OF_RANGE);
            for (int t = 0; t < K - 1; ++t) out[t * C] = nanv;
            continue;
        }
        float xb[2 * K - 2];
        float w[K];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) {
            xb[j] = load_f32(tails + (ti * (K - 1) + j) * C + c);
            xb[K - 1 + j] = load_f32(heads + (hi * (K - 1) + j) * C + c);
        }
#pragma unroll
        for (int j = 0; j < K; ++j) w[j] = a.weight[c * K + j];
        const float bias = a.bias ? a.bias[c] : 0.0f;
#pragma unroll
        for (int t = 0; t < K - 1; ++t) {
            float acc = bias;
#pragma unroll
            for (int j = 0; j < K; ++j) acc += w[j] * xb[t + j];
            if (a.activation == 1) acc = acc / (1.0f + expf(-acc));
            out[t * C] = acc;
        }
    }
}

template <typename XT>
hipError_t launch_k(const ConvArgs &a, dim3 grid, hipStream_t stream) {
    switch (a.ksize) {
    case 2: hipLaunchKernelGGL((conv_warmup_kernel<XT, 2>), grid, dim3(NT), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((conv_warmup_kernel<XT, 3>), grid, dim3(NT), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((conv_warmup_kernel<XT, 4>), grid, dim3(NT), 0, stream, a); break;
    case 5: hipLaunchKernelGGL((conv_warmup_kernel<XT, 5>), grid, dim3(NT), 0, stream, a); break;
    case 6: hipLaunchKernelGGL((conv_warmup_kernel<XT, 6>), grid, dim3(NT), 0, stream, a); break;
    case 7: hipLaunchKernelGGL((conv_warmup_kernel<XT, 7>), grid, dim3(NT), 0, stream, a); break;
    default: hipLaunchKernelGGL((conv_warmup_kernel<XT, 8>), grid, dim3(NT), 0, stream, a); break;
    }
    return hipGetLastError();
}

// 16-byte vector of inputs: 8 bf16 or 4 fp32 channels
template <typename XT> struct XVec;
template <> struct XVec<uint16_t> {
    static constexpr int N = 8;
    typedef uint4 raw;
    static __device__ __forceinline__ void unpack(raw r, float *f) {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct XVec<float> {
    static constexpr int N = 4;
    typedef float4 raw;
    static __device__ __forceinline__ void unpack(raw r, float *f) { f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w; }
};

template <typename XT, int K>
__global__ __launch_bounds__(NT) void conv_warmup_vec_kernel(ConvArgs a) {
    typedef XVec<XT> V;
    constexpr int NV = V::N;
    const int64_t C = a.channels;
    const int64_t c0 = ((int64_t)blockIdx.x * NT + threadIdx.x) * NV;
    if (c0 >= C) return;
    const XT *tails = static_cast<const XT *>(a.tails);
    const XT *heads = static_cast<const XT *>(a.heads);
    float w[NV][K];
#pragma unroll
    for (int i = 0; i < NV * K / 4; ++i) {
        const float4 q = *reinterpret_cast<const float4 *>(a.weight + c0 * K + 4 * i);
        const float qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) w[(4 * i + e) / K][(4 * i + e) % K] = qq[e];
    }
    float bias[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) bias[i] = a.bias ? a.bias[c0 + i] : 0.0f;
    const float nanv = __int_as_float(0x7fc00000);
    for (int64_t b = blockIdx.y; b < a.num_boundaries; b += gridDim.y) {
        const int64_t ti = a.tail_index ? a.tail_index[b] : b;
        const int64_t hi = a.head_index ? a.head_index[b] : b;
        float *out = a.out + b * (K - 1) * C + c0;
        if (ti < 0 || ti >= a.num_tails || hi < 0 || hi >= a.num_heads) {
            if (c0 == 0) raise_flag(a.err_flag, HYPIC_EFLAG_SLOT_OUT_OF_RANGE);
#pragma unroll
            for (int t = 0; t < K - 1; ++t)
#pragma unroll
                for (int i = 0; i < NV; i += 4)
                    *reinterpret_cast<float4 *>(out + t * C + i) = make_float4(nanv, nanv, nanv, nanv);
            continue;
        }
        typename V::raw r[2 * K - 2];
#pragma unroll
        for (int j = 0; j < K - 1; ++j) {
            r[j] = load_nt(reinterpret_cast<const typename V::raw *>(tails + (ti * (K - 1) + j) * C + c0));
            r[K - 1 + j] = load_nt(reinterpret_cast<const typename V::raw *>(heads + (hi * (K - 1) + j) * C + c0));
        }
        float xb[2 * K - 2][NV];
#pragma unroll
        for (int j = 0; j < 2 * K - 2; ++j) V::unpack(r[j], xb[j]);
#pragma unroll
        for (int t = 0; t < K - 1; ++t) {
            float y[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                float acc = bias[i];
#pragma unroll
                for (int j = 0; j < K; ++j) acc += w[i][j] * xb[t + j][i];
                if (a.activation == 1) acc = acc / (1.0f + expf(-acc));
                y[i] = acc;
            }
#pragma unroll
            for (int i = 0; i < NV; i += 4)
                __builtin_nontemporal_store((f32x4){y[i], y[i + 1], y[i + 2], y[i + 3]},
                                            reinterpret_cast<f32x4 *>(out + t * C + i));
        }
    }
}

template <typename XT>
hipError_t launch_vec_k(const ConvArgs &a, dim3 grid, hipStream_t stream) {
    switch (a.ksize) {
    case 2: hipLaunchKernelGGL((conv_warmup_vec_kernel<XT, 2>), grid, dim3(NT), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((conv_warmup_vec_kernel<XT, 3>), grid, dim3(NT), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((conv_warmup_vec_kernel<XT, 4>), grid, dim3(NT), 0, stream, a); break;
    case 5: hipLaunchKernelGGL((conv_warmup_vec_kernel<XT, 5>), grid, dim3(NT), 0, stream, a); break;
    case 6: hipLaunchKernelGGL((conv_warmup_vec_kernel<XT, 6>), grid, dim3(NT), 0, stream, a); break;
    case 7: hipLaunchKernelGGL((conv_warmup_vec_kernel<XT, 7>), grid, dim3(NT), 0, stream, a); break;
    default: hipLaunchKernelGGL((conv_warmup_vec_kernel<XT, 8>), grid, dim3(NT), 0, stream, a); break;
    }
    return hipGetLastError();
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

hipError_t launch_conv_warmup(const ConvArgs &a, hipStream_t stream) {
    if (a.num_boundaries <= 0) return hipSuccess;
    // vector kernel: 16 bytes of channels per thread; the weights of a thread's
    // channels (NV * K floats) must start 16-byte aligned too
    const int nv = a.x_dtype == HYPIC_BF16 ? 8 : 4;
    if (a.channels % nv == 0 && aligned16(a.tails) && aligned16(a.heads) && aligned16(a.out) &&
        aligned16(a.weight) && ((int64_t)nv * a.ksize) % 4 == 0 && (a.channels % 4 == 0)) {
        const int64_t gx = (a.channels / nv + NT - 1) / NT;
        const unsigned gy = (unsigned)(a.num_boundaries < 65535 ? a.num_boundaries : 65535);
        const dim3 grid((unsigned)gx, gy);
        if (a.x_dtype == HYPIC_BF16) return launch_vec_k<uint16_t>(a, grid, stream);
        return launch_vec_k<float>(a, grid, stream);
    }
    const int64_t total = (int64_t)a.num_boundaries * a.channels;
    int64_t blocks = (total + NT - 1) / NT;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) return hipSuccess;
    if (a.x_dtype == HYPIC_BF16) return launch_k<uint16_t>(a, dim3((unsigned)blocks), stream);
    return launch_k<float>(a, dim3((unsigned)blocks), stream);
}

}  // namespace hypic
