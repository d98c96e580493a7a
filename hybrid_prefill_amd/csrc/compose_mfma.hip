// Composition of GDN pool records on MFMA (d_k = d_v = 128).
//
// What it computes (besthub article "Cut First-Token Latency by 3.25x ...",
// paragraph 4: reuse composes T_C2*S(C1)+S(C2); podcast companion page,
// "Composition law, step by step"): per (request, head), over the chain in
// prompt order,
//     S <- e^{ell_i} (P_i S) + S_i
// and, in a second launch when the composed operator is asked for,
//     P <- P_i P        (P starts at I),   ell = sum_i ell_i.
//
// The chain is bandwidth-bound: every step streams one record (P_i and S_i,
// 128 KB) from HBM and does 4.2 MFLOP on it.  Accuracy needs more than one
// bf16 product (1e-4 relative for fp32 records), so P_i S is computed as
// hi.hi + hi.lo + lo.hi of the bf16 split x = hi + lo of both operands, which
// keeps about 16 significant bits and runs on the bf16 MFMA pipe.
//
// Work split: one 256-thread workgroup (4 waves) per (request, head).  Wave w
// keeps columns [32w, 32w+32) of the state as four fp32 32x32 accumulator
// tiles (rows 0-127).  P_i is staged once per step through LDS as bf16 hi/lo
// fragments laid out in MFMA operand order (one 16-byte read per lane, no bank
// conflicts); the B operand comes from the state's accumulator registers.  The
// next record is prefetched while the current product runs: P into registers
// (coalesced 16-byte loads), S straight from HBM into LDS (global_load_lds),
// read back from LDS in accumulator order.
#include "hypic_internal.h"

namespace hypic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

constexpr int D = 128;
constexpr int NT = 256;
constexpr int NFRAG = 4 * 8;          // (row block mb, k-step kb) fragments of P
// One fragment holds 64 lanes x 8 bf16 (4 dwords per lane).  Lane half h is
// placed 132 dwords after half 0 and fragments 264 dwords apart, so that the
// 8-byte staging writes of 16 consecutive threads (4 k-steps x 4 pieces) hit
// 16 distinct bank pairs, and the 16-byte operand reads stay conflict-free.
constexpr int FRAG_U32 = 264;
__device__ __forceinline__ int lane_slot(int li, int hh) { return 4 * li + 132 * hh; }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u16 bf_bits(float x) { return __builtin_bit_cast(u16, (__bf16)x); }
__device__ __forceinline__ float bf_val(u16 b) { return __uint_as_float((uint32_t)b << 16); }

// bf16 split x = hi + lo (both rounded to nearest even)
__device__ __forceinline__ void split(float x, u16 &hi, u16 &lo) {
    hi = bf_bits(x);
    lo = bf_bits(x - bf_val(hi));
}

__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// B operand from accumulator registers 8*half .. 8*half+7, as hi and lo parts
__device__ __forceinline__ void acc_to_b2(const f32x16 &c, int half, bf16x8 &bh, bf16x8 &bl) {
    u16 hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) split(c[8 * half + e], hi[e], lo[e]);
    u32x4 uh, ul;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uh[q] = (uint32_t)hi[2 * q] | ((uint32_t)hi[2 * q + 1] << 16);
        ul[q] = (uint32_t)lo[2 * q] | ((uint32_t)lo[2 * q + 1] << 16);
    }
    bh = __builtin_bit_cast(bf16x8, uh);
    bl = __builtin_bit_cast(bf16x8, ul);
}

// Fragment slot of P element (i, k): A operand of row block mb = i/32 and
// k-step kb, in the order that pairs with acc_to_b2 (k-step kb covers the
// 16 columns 16*kb .. 16*kb+15; lane half h takes columns 4h..4h+3 and
// 8+4h..8+4h+3 of them, as elements 0-3 and 4-7).
struct __align__(16) PStage {
    uint32_t hi[NFRAG * FRAG_U32];
    uint32_t lo[NFRAG * FRAG_U32];
    float s[D * D];                   // S_i, row-major, loaded straight from HBM into LDS
};

template <bool MODE_P>
__global__ __launch_bounds__(NT, 1) void compose_dense_mfma_kernel(ComposeArgs a) {
    __shared__ PStage ps;
    __shared__ int sh_bad;

    const int th = threadIdx.x;
    const int w = th >> 6, l = th & 63, h = l >> 5, l32 = l & 31;
    const int head = blockIdx.x % a.H;
    const int r = blockIdx.x / a.H;
    const int64_t orec = (int64_t)r * a.H + head;
    const int col0 = 32 * w;
    float *out = MODE_P ? a.out_P + orec * D * D : a.out_S + orec * D * D;

    // ---- chain validation (same rules as the reference kernel)
    if (th == 0) {
        const int64_t lo = a.chain_offsets[r], hi = a.chain_offsets[r + 1];
        sh_bad = (lo < 0 || hi < lo || hi > a.num_chain_slots) ? 2 : 0;
    }
    __syncthreads();
    const int64_t c_lo = a.chain_offsets[r], c_hi = a.chain_offsets[r + 1];
    if (sh_bad == 0) {
        __syncthreads();
        for (int64_t c = c_lo + th; c < c_hi; c += NT) {
            const int32_t s = a.chain_slots[c];
            if (s < 0 || s >= a.num_slots) sh_bad = 1;
        }
    }
    __syncthreads();
    const int bad = sh_bad;
    if (bad) {
        if (th == 0 && !MODE_P)
            raise_flag(a.err_flag, bad == 1 ? HYPIC_EFLAG_SLOT_OUT_OF_RANGE : HYPIC_EFLAG_BAD_OFFSETS);
        const float nanv = __int_as_float(0x7fc00000);
        for (int e = th; e < D * D; e += NT) out[e] = nanv;
        if (!MODE_P && a.out_ell && th == 0) a.out_ell[orec] = nanv;
        return;
    }

    // ---- initial state; the first record from a zero (S) or identity (P) start is taken as is
    f32x16 st[4];
    int64_t c = c_lo;
    const bool first_direct = MODE_P || a.init_S == nullptr;
    double ell = 0.0;
    if (first_direct && c < c_hi) {
        const int64_t rec = (int64_t)a.chain_slots[c] * a.H + head;
        const float *src = MODE_P ? a.pool_P + rec * D * D : a.pool_S + rec * D * D;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int q = 0; q < 16; ++q) st[mb][q] = src[(32 * mb + acc_row(q, h)) * D + col0 + l32];
        ell += (double)a.pool_ell[rec];
        ++c;
    } else {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = 32 * mb + acc_row(q, h);
                st[mb][q] = MODE_P ? (row == col0 + l32 ? 1.0f : 0.0f)
                                   : (a.init_S ? a.init_S[orec * D * D + (int64_t)row * D + col0 + l32] : 0.0f);
            }
    }

    // ---- P staging: thread th loads float4 pieces q = th + 256*u (u < 16) of P, row q/32,
    //      columns 4*(q%32) .. +3
    // both P_c and S_c are fetched as coalesced 16-byte pieces q = th + 256 u
    // P_c: coalesced 16-byte pieces q = th + 256 u into registers, split to bf16 hi/lo
    // fragments in LDS at the top of the step.  S_c: HBM -> LDS directly (no
    // registers), wave w's instruction u moving pieces (16 w + u) * 64 + lane.
    float4 pre[16];
#define HYPIC_FETCH_P(CC)                                                                        \
    do {                                                                                         \
        const int64_t frec = (int64_t)a.chain_slots[(CC)] * a.H + head;                          \
        const float4 *fsrc = reinterpret_cast<const float4 *>(a.pool_P + frec * D * D);          \
        _Pragma("unroll") for (int u = 0; u < 16; ++u) pre[u] = fsrc[th + NT * u];               \
    } while (0)
#define HYPIC_FETCH_S(CC)                                                                        \
    do {                                                                                         \
        const int64_t frec = (int64_t)a.chain_slots[(CC)] * a.H + head;                          \
        const float4 *fss = reinterpret_cast<const float4 *>(a.pool_S + frec * D * D);           \
        _Pragma("unroll") for (int u = 0; u < 16; ++u)                                           \
            __builtin_amdgcn_global_load_lds(fss + (16 * w + u) * 64 + l,                       \
                                             &ps.s[(16 * w + u) * 256], 16, 0, 0);               \
    } while (0)
    if (c < c_hi) {
        HYPIC_FETCH_P(c);
        if (!MODE_P) HYPIC_FETCH_S(c);
    }

    for (; c < c_hi; ++c) {
        const int64_t rec = (int64_t)a.chain_slots[c] * a.H + head;
        // stage P_c (bf16 hi/lo, fragment order)
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int q = th + NT * u;
            const int i = q >> 5, k0 = 4 * (q & 31);
            const int mb = i >> 5, li = i & 31;
            const int kb = k0 >> 4, c16 = k0 & 15;
            const int hh = (c16 >> 2) & 1, e0 = (c16 >> 3) * 4;
            u16 hi[4], lo[4];
            split(pre[u].x, hi[0], lo[0]);
            split(pre[u].y, hi[1], lo[1]);
            split(pre[u].z, hi[2], lo[2]);
            split(pre[u].w, hi[3], lo[3]);
            const int slot = (mb * 8 + kb) * FRAG_U32 + lane_slot(li, hh) + (e0 >> 1);
            *reinterpret_cast<u32x2 *>(&ps.hi[slot]) =
                u32x2{(uint32_t)hi[0] | ((uint32_t)hi[1] << 16), (uint32_t)hi[2] | ((uint32_t)hi[3] << 16)};
            *reinterpret_cast<u32x2 *>(&ps.lo[slot]) =
                u32x2{(uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16)};
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");    // this wave's S_c pieces have landed
        __syncthreads();
        float sadd[4][16];
        if (!MODE_P) {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int q = 0; q < 16; ++q) sadd[mb][q] = ps.s[(32 * mb + acc_row(q, h)) * D + col0 + l32];
            __syncthreads();                                   // S_c read by all before S_{c+1} lands
        }
        if (c + 1 < c_hi) {                                    // the next record flies during this product
            HYPIC_FETCH_P(c + 1);
            if (!MODE_P) HYPIC_FETCH_S(c + 1);
        }
        const float le = a.pool_ell[rec];
        // acc = P_c * state, hi.hi + hi.lo + lo.hi
        // the state's B fragments (hi, lo) for all 8 k-steps, once per step; the
        // state itself is not needed again until the combine overwrites it
        bf16x8 bh[8], bl[8];
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) acc_to_b2(st[kb >> 1], kb & 1, bh[kb], bl[kb]);
        f32x16 acc[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[mb][q] = 0.f;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            bf16x8 ah[4], al[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int f = (mb * 8 + kb) * FRAG_U32 + lane_slot(l32, h);
                ah[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&ps.hi[f]));
                al[mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&ps.lo[f]));
            }
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma(ah[mb], bh[kb], acc[mb]);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma(ah[mb], bl[kb], acc[mb]);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma(al[mb], bh[kb], acc[mb]);
        }
        if (MODE_P) {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) st[mb] = acc[mb];
        } else {
            const float sc = expf(le);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int q = 0; q < 16; ++q) st[mb][q] = sc * acc[mb][q] + sadd[mb][q];
        }
        ell += (double)le;
        __syncthreads();     // everyone is done with this P before the next is staged
    }
#undef HYPIC_FETCH_P
#undef HYPIC_FETCH_S
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q = 0; q < 16; ++q) out[(int64_t)(32 * mb + acc_row(q, h)) * D + col0 + l32] = st[mb][q];
    if (!MODE_P && a.out_ell && th == 0) a.out_ell[orec] = (float)ell;
}

}  // namespace

hipError_t launch_compose_mfma(const ComposeArgs &a, hipStream_t stream, bool *taken) {
    *taken = false;
    if (a.family != HYPIC_GDN || a.dk != 128 || a.dv != 128) return hipSuccess;
    *taken = true;
    const dim3 grid((unsigned)((int64_t)a.num_requests * a.H));
    hipLaunchKernelGGL(compose_dense_mfma_kernel<false>, grid, dim3(NT), 0, stream, a);
    if (a.out_P) hipLaunchKernelGGL(compose_dense_mfma_kernel<true>, grid, dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace hypic
