// Measured-peak microbenchmarks (libhypic_peaks.so, used by the benchmark only; not
// part of the hot path's C ABI in include/hypic.h).  The benchmark reports every
// kernel against the published MI355X peaks; these two kernels measure what this
// box delivers under the same conditions, so that the fractions can also be read
// against attainable rates:
//   * a streaming read of a large buffer (16-byte non-temporal loads, four in flight
//     per thread, grid-stride), the attainable HBM read bandwidth;
//   * a streaming copy (the same loads, each followed by a 16-byte non-temporal
//     store), the attainable rate of a kernel that writes as much as it reads;
//   * a loop of independent bf16 v_mfma_f32_32x32x16 products on register operands
//     (four accumulator chains per wave, one wave per SIMD), the attainable dense
//     bf16 matrix rate at the clock the chip holds under that load.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int NT = 256;
constexpr int NT_READ = 512;

__global__ __launch_bounds__(NT_READ) void peak_read_kernel(const f32x4 *src, int64_t n4, float *sink) {
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, acc2 = acc0, acc3 = acc0;
    const int64_t stride = (int64_t)gridDim.x * NT_READ;
    int64_t i = (int64_t)blockIdx.x * NT_READ + threadIdx.x;
    for (; i + 3 * stride < n4; i += 4 * stride) {
        acc0 += __builtin_nontemporal_load(src + i);
        acc1 += __builtin_nontemporal_load(src + i + stride);
        acc2 += __builtin_nontemporal_load(src + i + 2 * stride);
        acc3 += __builtin_nontemporal_load(src + i + 3 * stride);
    }
    for (; i < n4; i += stride) acc0 += __builtin_nontemporal_load(src + i);
    const f32x4 acc = acc0 + acc1 + acc2 + acc3;
    const float s = acc.x + acc.y + acc.z + acc.w;
    // a store that never happens for finite data keeps every load live
    if (s != s) sink[blockIdx.x] = s;
}

__global__ __launch_bounds__(NT_READ) void peak_copy_kernel(const f32x4 *src, f32x4 *dst, int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * NT_READ;
    int64_t i = (int64_t)blockIdx.x * NT_READ + threadIdx.x;
    for (; i + 3 * stride < n4; i += 4 * stride) {
        const f32x4 a0 = __builtin_nontemporal_load(src + i);
        const f32x4 a1 = __builtin_nontemporal_load(src + i + stride);
        const f32x4 a2 = __builtin_nontemporal_load(src + i + 2 * stride);
        const f32x4 a3 = __builtin_nontemporal_load(src + i + 3 * stride);
        __builtin_nontemporal_store(a0, dst + i);
        __builtin_nontemporal_store(a1, dst + i + stride);
        __builtin_nontemporal_store(a2, dst + i + 2 * stride);
        __builtin_nontemporal_store(a3, dst + i + 3 * stride);
    }
    for (; i < n4; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(NT) void peak_mfma_kernel(int64_t iters, float *sink) {
    const float x = 1.0f + 1e-3f * (float)(threadIdx.x & 7);
    const bf16x8 a = {(__bf16)x, (__bf16)x, (__bf16)x, (__bf16)x, (__bf16)x, (__bf16)x, (__bf16)x, (__bf16)x};
    const bf16x8 b = a;
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int64_t i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    const f32x16 c = c0 + c1 + c2 + c3;
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[r];
    if (s != s) sink[blockIdx.x * NT + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Streaming read of `bytes` (a multiple of 16) from `src` by `blocks` workgroups of
// 512 threads; sink: one float per block (never written for finite data).  Returns 0, or -1 on a bad argument / launch error.
int hypic_peak_read(const void *src, int64_t bytes, int32_t blocks, float *sink, void *stream) {
    if (!src || !sink || bytes <= 0 || (bytes & 15) || blocks <= 0) return -1;
    hipLaunchKernelGGL(peak_read_kernel, dim3((unsigned)blocks), dim3(NT_READ), 0, static_cast<hipStream_t>(stream),
                       static_cast<const f32x4 *>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Streaming copy of `bytes` (a multiple of 16) from `src` to `dst` (not overlapping)
// by `blocks` workgroups of 512 threads.  Returns 0, or -1 on a bad argument / launch error.
int hypic_peak_copy(const void *src, void *dst, int64_t bytes, int32_t blocks, void *stream) {
    if (!src || !dst || bytes <= 0 || (bytes & 15) || blocks <= 0) return -1;
    hipLaunchKernelGGL(peak_copy_kernel, dim3((unsigned)blocks), dim3(NT_READ), 0, static_cast<hipStream_t>(stream),
                       static_cast<const f32x4 *>(src), static_cast<f32x4 *>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// `blocks` workgroups of four waves, each wave `iters` x 4 products of 32x32x16
// (32768 FLOP each); sink: one float per thread (never written).
int hypic_peak_mfma(int64_t iters, int32_t blocks, float *sink, void *stream) {
    if (!sink || iters <= 0 || blocks <= 0) return -1;
    hipLaunchKernelGGL(peak_mfma_kernel, dim3((unsigned)blocks), dim3(NT), 0, static_cast<hipStream_t>(stream),
                       iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
