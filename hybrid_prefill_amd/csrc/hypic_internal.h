// Internal declarations shared by the HIP translation units of libhypic.
// Not part of the public ABI (include/hypic.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hypic.h"

namespace hypic {

// Kernel-side view of one build call (all device pointers).
struct BuildArgs {
    int32_t family, H, dk, dv, num_segments, kv_dtype;
    int64_t num_tokens;
    const int64_t *seg_offsets;
    const void *k;  int64_t k_st, k_sh;
    const void *v;  int64_t v_st, v_sh;
    const float *beta; int64_t b_st, b_sh;
    const float *log_alpha; int64_t la_st, la_sh;
    const int32_t *dst_slots;
    int64_t num_slots;
    float *pool_ell, *pool_P, *pool_S;
    uint32_t *err_flag;
};

struct ComposeArgs {
    int32_t family, H, dk, dv, num_requests;
    int64_t num_slots, num_chain_slots;
    const float *pool_ell, *pool_P, *pool_S;
    const int64_t *chain_offsets;
    const int32_t *chain_slots;
    const float *init_S;
    float *out_S, *out_ell, *out_P;
    uint32_t *err_flag;
    // per chain entry, tokens applied to the state before its record (NULL: none)
    const int64_t *head_offsets;        // [num_chain_slots + 1]
    const float *head_k, *head_v;       // [T][H][d_k], [T][H][d_v]
    const float *head_beta, *head_la;   // [T][H]
    int64_t num_head_tokens;            // T
};

struct ConvArgs {
    int32_t num_boundaries, channels, ksize, x_dtype, activation;
    const void *tails; int64_t num_tails; const int32_t *tail_index;
    const void *heads; int64_t num_heads; const int32_t *head_index;
    const float *weight, *bias;
    float *out;
    uint32_t *err_flag;
};

struct ConvKvArgs {
    int32_t num_tokens, H, dk, dv, ksize, x_dtype, activation, normalize_k, out_dtype;
    const void *x; int64_t num_rows;
    const int32_t *window;
    const float *weight, *bias;
    void *k_out, *v_out;
    const int32_t *src_token; int64_t num_src_tokens;
    const float *beta, *log_alpha;
    float *beta_out, *la_out;
    uint32_t *err_flag;
};

// Queries and in-segment outputs of the chunked prefill forward (device pointers,
// strides in elements): q in the keys' dtype, o fp32 or bf16 (o_bf16).
struct FwdIO {
    const void *q; int64_t q_st, q_sh;
    void *o; int64_t o_st, o_sh;
    int32_t o_bf16;
};

hipError_t launch_build(const BuildArgs &a, hipStream_t stream);
hipError_t launch_chunk_mfma(const BuildArgs &a, const FwdIO &io, bool records, bool outputs, hipStream_t stream,
                             bool *taken);
hipError_t launch_compose(const ComposeArgs &a, hipStream_t stream);
hipError_t launch_conv_warmup(const ConvArgs &a, hipStream_t stream);
hipError_t launch_conv_kv(const ConvKvArgs &a, hipStream_t stream);
hipError_t launch_build_kda_mfma(const BuildArgs &a, hipStream_t stream);

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

template <typename T> __device__ __forceinline__ float load_f32(const T *p);
template <> __device__ __forceinline__ float load_f32<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float load_f32<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

// Cache policy of loads that stream data read once (records, keys, values, conv
// inputs): the non-temporal bit (the aux/cpol operand's value 2 on gfx950, printed
// "nt").  Such lines are not kept in the L2 and the Infinity Cache at the expense
// of data that is reused; streaming reads of HBM run at about 7 TB/s with it
// against about 6.3 TB/s without.
constexpr int kLoadNT = 2;

// Word 3 of a raw buffer resource (__builtin_amdgcn_make_buffer_rsrc): the 32-bit
// data format, as for every gfx9 buffer access.
constexpr int RSRC_WORD3 = 0x00020000;

template <typename T> __device__ __forceinline__ T load_nt(const T *p) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    static_assert(sizeof(T) == 16 || sizeof(T) == 8, "8- or 16-byte loads only");
    if constexpr (sizeof(T) == 16)
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p)));
    else
        return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p)));
}

__device__ __forceinline__ void raise_flag(uint32_t *flag, uint32_t bits) {
    if (flag) atomicOr(flag, bits);
}

// HBM -> LDS loads that the compiler does not see (global_load_lds through inline
// asm, non-temporal; lane i of the wave lands its bytes at dst + size * i, dst
// uniform over the wave).  The compiler's wait counting does not order such DMA
// loads with loads into registers: after a global_load_lds it waits for every
// load in flight (vmcnt(0)) before it uses any register loaded earlier, and before
// any LDS read that may alias the DMA's target.  Hidden from it, the DMA loads
// still count in the hardware's in-order counter, so the compiler's own waits for
// register loads only ever wait for more, never less; the kernel then waits for
// its DMA data itself (s_waitcnt vmcnt(n) with n the loads it issued after them).
__device__ __forceinline__ uint32_t lds_off(const void *p) {
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p);
}
__device__ __forceinline__ void lds_dma16(const void *src, void *dst) {
    uint32_t keep;     // m0 is the compiler's: restored after the load
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep)
                 : "v"(src), "s"(lds_off(dst))
                 : "memory");
}
// the same without the non-temporal policy: for an operand that another workgroup of
// the same XCD reads too, which should find it in the L2
__device__ __forceinline__ void lds_dma16_shared(const void *src, void *dst) {
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep)
                 : "v"(src), "s"(lds_off(dst))
                 : "memory");
}
__device__ __forceinline__ void lds_dma4(const void *src, void *dst) {
    uint32_t keep;     // m0 is the compiler's: restored after the load
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off nt\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep)
                 : "v"(src), "s"(lds_off(dst))
                 : "memory");
}

// Workgroup barrier that orders LDS only: the wave's ds_* operations complete before
// it arrives; outstanding vector-memory loads (prefetches into registers, and
// global_load_lds whose data is consumed later and waited for explicitly by vmcnt)
// keep flying.  __syncthreads's workgroup-scope fence would wait for all of them.
// The memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace hypic
