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
// Bandwidth-bound: each thread owns one channel of one boundary and reads its
// 2(K-1) inputs and K weights; consecutive threads take consecutive channels,
// so every load and store is coalesced along C.
#include "hypic_internal.h"

namespace hypic {
namespace {

constexpr int NT = 256;

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

}  // namespace

hipError_t launch_conv_warmup(const ConvArgs &a, hipStream_t stream) {
    const int64_t total = (int64_t)a.num_boundaries * a.channels;
    int64_t blocks = (total + NT - 1) / NT;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) return hipSuccess;
    if (a.x_dtype == HYPIC_BF16) return launch_k<uint16_t>(a, dim3((unsigned)blocks), stream);
    return launch_k<float>(a, dim3((unsigned)blocks), stream);
}

}  // namespace hypic
