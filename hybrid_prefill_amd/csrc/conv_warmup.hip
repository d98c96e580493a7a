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
// Bandwidth-bound.  Main kernel: the boundaries are the grid's y index (their
// table indices are wave-uniform scalar loads) and each thread owns four channels
// of every row, so every load is one 8- or 16-byte access and every output row one
// 16-byte store, coalesced along C.  Channel counts or pointers that do not allow
// that take the one-channel-per-thread kernel.
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

// Four channels of one input row: 8 bytes of bf16 or 16 bytes of fp32
template <typename XT> struct XVec;
template <> struct XVec<uint16_t> {
    typedef uint2 raw;
    static __device__ __forceinline__ void unpack(raw r, float *f) {
        f[0] = __uint_as_float(r.x << 16);
        f[1] = __uint_as_float(r.x & 0xffff0000u);
        f[2] = __uint_as_float(r.y << 16);
        f[3] = __uint_as_float(r.y & 0xffff0000u);
    }
};
template <> struct XVec<float> {
    typedef float4 raw;
    static __device__ __forceinline__ void unpack(raw r, float *f) { f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w; }
};

// Each thread owns four channels, so that every output row is one 16-byte store per
// lane over a contiguous kilobyte per wave (eight bf16 channels per thread would
// take two stores per row at a 32-byte stride, half a sector each: about 1.5x
// slower).  A workgroup takes NB boundaries per pass and issues all their loads
// before the first one is used.
constexpr int CONV_NB = 2;

template <typename XT, int K>
__global__ __launch_bounds__(NT) void conv_warmup_vec_kernel(ConvArgs a) {
    typedef XVec<XT> V;
    const int64_t C = a.channels;
    const int64_t c0 = ((int64_t)blockIdx.x * NT + threadIdx.x) * 4;
    if (c0 >= C) return;
    const XT *tails = static_cast<const XT *>(a.tails);
    const XT *heads = static_cast<const XT *>(a.heads);
    float w[4][K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const float4 q = *reinterpret_cast<const float4 *>(a.weight + c0 * K + 4 * i);
        const float qq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) w[(4 * i + e) / K][(4 * i + e) % K] = qq[e];
    }
    float bias[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) bias[i] = a.bias ? a.bias[c0 + i] : 0.0f;
    const float nanv = __int_as_float(0x7fc00000);
    const int64_t nb = a.num_boundaries;
    for (int64_t b0 = (int64_t)blockIdx.y * CONV_NB; b0 < nb; b0 += (int64_t)gridDim.y * CONV_NB) {
        typename V::raw r[CONV_NB][2 * K - 2];
        bool ok[CONV_NB];
#pragma unroll
        for (int u = 0; u < CONV_NB; ++u) {
            const int64_t b = b0 + u < nb ? b0 + u : nb - 1;
            const int64_t ti = a.tail_index ? a.tail_index[b] : b;
            const int64_t hi = a.head_index ? a.head_index[b] : b;
            ok[u] = ti >= 0 && ti < a.num_tails && hi >= 0 && hi < a.num_heads;
            if (ok[u]) {                            // uniform over the workgroup
#pragma unroll
                for (int j = 0; j < K - 1; ++j) {
                    r[u][j] = load_nt(reinterpret_cast<const typename V::raw *>(tails + (ti * (K - 1) + j) * C + c0));
                    r[u][K - 1 + j] =
                        load_nt(reinterpret_cast<const typename V::raw *>(heads + (hi * (K - 1) + j) * C + c0));
                }
            }
        }
#pragma unroll
        for (int u = 0; u < CONV_NB; ++u) {
            const int64_t b = b0 + u;
            if (b >= nb) break;
            float *out = a.out + b * (K - 1) * C + c0;
            if (!ok[u]) {
                if (c0 == 0) raise_flag(a.err_flag, HYPIC_EFLAG_SLOT_OUT_OF_RANGE);
#pragma unroll
                for (int t = 0; t < K - 1; ++t)
                    *reinterpret_cast<float4 *>(out + t * C) = make_float4(nanv, nanv, nanv, nanv);
                continue;
            }
            float xb[2 * K - 2][4];
#pragma unroll
            for (int j = 0; j < 2 * K - 2; ++j) V::unpack(r[u][j], xb[j]);
#pragma unroll
            for (int t = 0; t < K - 1; ++t) {
                float y[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float acc = bias[i];
#pragma unroll
                    for (int j = 0; j < K; ++j) acc += w[i][j] * xb[t + j][i];
                    if (a.activation == 1) acc = acc / (1.0f + expf(-acc));
                    y[i] = acc;
                }
                __builtin_nontemporal_store((f32x4){y[0], y[1], y[2], y[3]}, reinterpret_cast<f32x4 *>(out + t * C));
            }
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
    // vector kernel: four channels per thread (8- or 16-byte loads, 16-byte stores);
    // the weights of a thread's channels (4 K floats) start 16-byte aligned too
    if (a.channels % 4 == 0 && aligned16(a.tails) && aligned16(a.heads) && aligned16(a.out) &&
        aligned16(a.weight)) {
        const int64_t gx = (a.channels / 4 + NT - 1) / NT;
        const int64_t passes = (a.num_boundaries + CONV_NB - 1) / CONV_NB;
        const unsigned gy = (unsigned)(passes < 65535 ? passes : 65535);
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
