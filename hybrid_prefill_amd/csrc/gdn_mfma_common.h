// Helpers shared by the GDN chunk kernels on MFMA (d_k = d_v = 128, bf16 operands,
// fp32 accumulation): operand packing and layouts of v_mfma_f32_32x32x16_bf16, the
// wave prefix sum, and the per-chunk factor preparation (Gram blocks, the blocked
// inversion of I + A0 and the K^T turnaround).  The formulas and the layout facts
// are stated where they are used: build_mfma.hip (records) and build_fwd_mfma.hip
// (records and in-segment outputs).  Each including translation unit gets its own
// copy (internal linkage).
//
// The Smem-dependent helpers are templates on the kernel's LDS layout SM, which
// provides Km, Kt, TB, H21, Af, pv, inv_tmp, the flag kWithP (false: the P system is
// not built, its factors are not written) and kS, the system index of the S factors
// in TB and H21 (the P factors are at index 0 when they exist).
#pragma once

#include <atomic>

#include "hypic_internal.h"

namespace hypic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

constexpr int CH = 64;     // tokens per chunk
constexpr int D = 128;     // d_k = d_v
constexpr int KML = 128;   // row length (bf16) of Km, Vm [token][channel], granules swizzled (kmo)
constexpr int KTL = 72;    // row length (bf16) of Kt [channel][token]
constexpr int AFL = 36;    // row length (fp32) of the 32x32 diagonal blocks in Af
constexpr int TBL = 40;    // row length (bf16) of the 32x32 factor tiles


// Km, Vm: 16-byte granule g of row t sits in slot g ^ (t % 16) of the row, so the 16
// rows one MFMA operand read touches hit 16 different slots (no bank conflicts)
// without padding, which lets global_load_lds fill the rows directly.
__device__ __forceinline__ int kmo(int t, int g) { return t * KML + ((g ^ (t & 15)) << 3); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u16 f2bf(float x) { return __builtin_bit_cast(u16, (__bf16)x); }

// fp32 -> bf16 (round to nearest even), two values per v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                        float a7) {
    return __builtin_convertvector((f32x8){a0, a1, a2, a3, a4, a5, a6, a7}, bf16x8);
}

__device__ __forceinline__ s16x4 pack4(float a0, float a1, float a2, float a3) {
    return __builtin_bit_cast(s16x4, __builtin_convertvector((f32x4){a0, a1, a2, a3}, bf16x4));
}

// 8 consecutive bf16 from LDS (16-byte aligned)
__device__ __forceinline__ bf16x8 lds8(const u16 *p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}

// Order this wave's LDS writes before its later LDS reads (the lanes of a wave
// run in lockstep, so no workgroup barrier is needed when only this wave reads).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele inside each row
// of 16 lanes (DPP row shifts, zero fill), then the row totals via the row
// broadcasts of lane 15 (to rows 1, 3) and lane 31 (to rows 2, 3).
#define HYPIC_DPP_ADD(X, CTRL, ROWMASK) \
    X += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(X), CTRL, ROWMASK, 0xf, true))
__device__ __forceinline__ float wave_prefix_sum(float x) {
    HYPIC_DPP_ADD(x, 0x111, 0xf);    // row_shr:1
    HYPIC_DPP_ADD(x, 0x112, 0xf);    // row_shr:2
    HYPIC_DPP_ADD(x, 0x114, 0xf);    // row_shr:4
    HYPIC_DPP_ADD(x, 0x118, 0xf);    // row_shr:8
    HYPIC_DPP_ADD(x, 0x142, 0xa);    // row_bcast:15
    HYPIC_DPP_ADD(x, 0x143, 0xc);    // row_bcast:31
    return x;
}
#undef HYPIC_DPP_ADD

// Row of the 32x32 accumulator element held in register r by lane half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// B operand (k-step `half` of a 32-row block) from accumulator registers.
__device__ __forceinline__ bf16x8 acc_to_b(const f32x16 &c, int half) {
    const int o = 8 * half;
    return pack8(c[o + 0], c[o + 1], c[o + 2], c[o + 3], c[o + 4], c[o + 5], c[o + 6], c[o + 7]);
}

// Bits 2 and 3 swapped (an involution).
__device__ __forceinline__ int swz(int c) { return (c & ~12) | ((c & 4) << 1) | ((c & 8) >> 1); }

// B operand of the identity for k-step ks (column l32, rows 16 ks + 8h + e): at most
// one element is 1.0 (bf16 0x3f80), element d = l32 - 16 ks - 8h when 0 <= d < 8.
__device__ __forceinline__ bf16x8 eye_b(int ks, int h, int l32) {
    const int d = l32 - 16 * ks - 8 * h;
    const uint32_t one = (unsigned)d < 8u ? 0x3f80u << (16 * (d & 1)) : 0u;
    const int wd = d >> 1;
    const u32x4 u = {wd == 0 ? one : 0u, wd == 1 ? one : 0u, wd == 2 ? one : 0u, wd == 3 ? one : 0u};
    return __builtin_bit_cast(bf16x8, u);
}

// Per-token values for registers 4q..4q+3 of a swizzled accumulator tile whose
// physical rows 32 mb + 8q + 4h + 0..3 hold tokens 32 mb + 16 (q/2) + 8h + 4 (q%2) + 0..3.
__device__ __forceinline__ float4 tok4(const float *v, int mb, int q, int h) {
    return *reinterpret_cast<const float4 *>(v + 32 * mb + 16 * (q >> 1) + 8 * h + 4 * (q & 1));
}

// Prep wave pw (1 or 3): the inverse factors of 32x32 diagonal block `blk` for
// both systems from A0_blk in Af.  With D = diag(e^g), A = D A0 D^{-1}, so
// (I + A)^{-1} = D (I + A0)^{-1} D^{-1}: one fp32 inversion T0 of I + A0_blk
// serves both, entry (r, c) of the S inverse being T0[r][c] e^{g_r - g_c}.
// T0 is built in place in Af (4x4 blocks in closed form, merges to 8 and 16 in
// fp32, the merge to 32 on the MFMA); each level writes its part of
// -T0 diag(beta) (P) and D T0 D^{-1} diag(beta) (S) into TB[par] in bf16.
// TB's upper triangles are zeroed once per segment and never written here.
// Part 1 (level 0) runs in phase a right after the Gram block, part 2 (levels 1
// and 2 and the merge) in phase b; TB is double-buffered by chunk parity, so
// the writes may land while the state waves read the previous chunk's factors.
// bs (optional): per-column factors of the S tile, which is then T0 diag(bs) (a row
// scaling of the S system's solve folded into it, see the record build) instead of
// D T0 D^{-1} diag(beta).
struct InvCtx {
    float *M, *tmp;
    u16 *TP, *TS;
    const float *bet, *gg, *bs;
};

template <class SM>
__device__ __forceinline__ InvCtx inv_ctx(SM &sm, int par, int blk, int pw, const float *bs = nullptr) {
    return InvCtx{sm.Af[blk], sm.inv_tmp[pw], sm.TB[par][0][blk], sm.TB[par][SM::kS][blk], &sm.pv[pw][1][32 * blk],
                  &sm.pv[pw][0][32 * blk], bs};
}

// both factors of one T0 entry x at (r, c), r > c (WP = false: the S factor only)
template <bool WP>
__device__ __forceinline__ void inv_put(const InvCtx &v, int r, int c, float x) {
    const float bx = x * v.bet[c];
    if (WP) v.TP[r * TBL + c] = f2bf(-bx);
    v.TS[r * TBL + c] = f2bf(v.bs ? x * v.bs[c] : bx * __expf(v.gg[r] - v.gg[c]));
}

// both factors of four consecutive T0 entries of row r, columns c .. c + 3
// (entries above the diagonal are zero in T0 and written as zero)
template <bool WP>
__device__ __forceinline__ void inv_put4(const InvCtx &v, int r, int c, float4 x) {
    const float4 b4 = *reinterpret_cast<const float4 *>(&v.bet[c]);
    const float4 g4 = *reinterpret_cast<const float4 *>(&v.gg[c]);
    const float gr = v.gg[r];
    const float b0 = x.x * b4.x, b1 = x.y * b4.y, b2 = x.z * b4.z, b3 = x.w * b4.w;
    if (WP) *reinterpret_cast<u32x2 *>(&v.TP[r * TBL + c]) = u32x2{pack2(-b0, -b1), pack2(-b2, -b3)};
    if (v.bs) {
        const float4 s4 = *reinterpret_cast<const float4 *>(&v.bs[c]);
        const float s0 = r >= c ? x.x * s4.x : 0.f, s1 = r >= c + 1 ? x.y * s4.y : 0.f;
        const float s2 = r >= c + 2 ? x.z * s4.z : 0.f, s3 = r >= c + 3 ? x.w * s4.w : 0.f;
        *reinterpret_cast<u32x2 *>(&v.TS[r * TBL + c]) = u32x2{pack2(s0, s1), pack2(s2, s3)};
        return;
    }
    const float e0 = r >= c ? __expf(gr - g4.x) : 0.f, e1 = r >= c + 1 ? __expf(gr - g4.y) : 0.f;
    const float e2 = r >= c + 2 ? __expf(gr - g4.z) : 0.f, e3 = r >= c + 3 ? __expf(gr - g4.w) : 0.f;
    *reinterpret_cast<u32x2 *>(&v.TS[r * TBL + c]) = u32x2{pack2(b0 * e0, b1 * e1), pack2(b2 * e2, b3 * e3)};
}

template <bool WP>
__device__ __forceinline__ void prep_invert1(const InvCtx &v, int l) {
    float *M = v.M;
    if (l < 32) {
        // level 0: the 4x4 diagonal block o = 16 (l / 16) + 4 ((l / 4) % 4) in closed form;
        // lane row i = l % 4
        const int o = 16 * (l >> 4) + 4 * ((l >> 2) & 3), i = l & 3;
        const float n10 = M[(o + 1) * AFL + o];
        const float n20 = M[(o + 2) * AFL + o], n21 = M[(o + 2) * AFL + o + 1];
        const float n30 = M[(o + 3) * AFL + o], n31 = M[(o + 3) * AFL + o + 1], n32 = M[(o + 3) * AFL + o + 2];
        const float t20 = n21 * n10 - n20, t31 = n32 * n21 - n31;
        const float t30 = -n30 + n31 * n10 - n32 * t20;
        float4 x;
        x.x = i == 0 ? 1.f : i == 1 ? -n10 : i == 2 ? t20 : t30;
        x.y = i == 0 ? 0.f : i == 1 ? 1.f : i == 2 ? -n21 : t31;
        x.z = i < 2 ? 0.f : i == 2 ? 1.f : -n32;
        x.w = i == 3 ? 1.f : 0.f;
        *reinterpret_cast<float4 *>(&M[(o + i) * AFL + o]) = x;
        inv_put4<WP>(v, o + i, o, x);
    }
    wave_lds_sync();
}

template <bool WP>
__device__ __forceinline__ void prep_invert2(const InvCtx &v, int l) {
    float *M = v.M, *tmp = v.tmp;
    {
        // level 1 (4 -> 8): T_10 = -T_11 (A_10 T_00); merge m = l / 16 at
        // o = 16 (m / 2) + 8 (m % 2); output (i, j) of the 4x4 block T_10 at rows
        // o + 4 + i, columns o + j
        const int m = l >> 4, o = 16 * (m >> 1) + 8 * (m & 1), i = (l >> 2) & 3, j = l & 3;
        const float4 n = *reinterpret_cast<const float4 *>(&M[(o + 4 + i) * AFL + o]);
        const float t = n.x * M[o * AFL + o + j] + n.y * M[(o + 1) * AFL + o + j] + n.z * M[(o + 2) * AFL + o + j] +
                        n.w * M[(o + 3) * AFL + o + j];
        tmp[16 * m + 4 * i + j] = t;
        wave_lds_sync();
        const float4 t11 = *reinterpret_cast<const float4 *>(&M[(o + 4 + i) * AFL + o + 4]);
        const float x = -(t11.x * tmp[16 * m + j] + t11.y * tmp[16 * m + 4 + j] + t11.z * tmp[16 * m + 8 + j] +
                          t11.w * tmp[16 * m + 12 + j]);
        M[(o + 4 + i) * AFL + o + j] = x;
        inv_put<WP>(v, o + 4 + i, o + j, x);
    }
    wave_lds_sync();
    {
        // level 2 (8 -> 16): merge m = l / 32 at R = 16 m; lane outputs (i, j), (i, j + 1)
        // of the 8x8 block T_10 at rows R + 8 + i, columns R + j
        const int m = l >> 5, R = 16 * m, i = (l & 31) >> 2, j = 2 * (l & 3);
        const float4 na = *reinterpret_cast<const float4 *>(&M[(R + 8 + i) * AFL + R]);
        const float4 nb = *reinterpret_cast<const float4 *>(&M[(R + 8 + i) * AFL + R + 4]);
        const float nv[8] = {na.x, na.y, na.z, na.w, nb.x, nb.y, nb.z, nb.w};
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float2 tk = *reinterpret_cast<const float2 *>(&M[(R + k) * AFL + R + j]);
            t0 += nv[k] * tk.x;
            t1 += nv[k] * tk.y;
        }
        *reinterpret_cast<float2 *>(&tmp[64 * m + 8 * i + j]) = make_float2(t0, t1);
        wave_lds_sync();
        const float4 ta = *reinterpret_cast<const float4 *>(&M[(R + 8 + i) * AFL + R + 8]);
        const float4 tb = *reinterpret_cast<const float4 *>(&M[(R + 8 + i) * AFL + R + 12]);
        const float tv[8] = {ta.x, ta.y, ta.z, ta.w, tb.x, tb.y, tb.z, tb.w};
        float u0 = 0.f, u1 = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float2 c = *reinterpret_cast<const float2 *>(&tmp[64 * m + 8 * k + j]);
            u0 += tv[k] * c.x;
            u1 += tv[k] * c.y;
        }
        *reinterpret_cast<float2 *>(&M[(R + 8 + i) * AFL + R + j]) = make_float2(-u0, -u1);
        const int r = R + 8 + i, c = R + j;
        const float2 b2 = *reinterpret_cast<const float2 *>(&v.bet[c]);
        const float2 g2 = *reinterpret_cast<const float2 *>(&v.gg[c]);
        const float gr = v.gg[r];
        const float b0 = -u0 * b2.x, b1 = -u1 * b2.y;
        if (WP) *reinterpret_cast<uint32_t *>(&v.TP[r * TBL + c]) = pack2(-b0, -b1);
        if (v.bs) {
            const float2 s2 = *reinterpret_cast<const float2 *>(&v.bs[c]);
            *reinterpret_cast<uint32_t *>(&v.TS[r * TBL + c]) = pack2(-u0 * s2.x, -u1 * s2.y);
        } else {
            *reinterpret_cast<uint32_t *>(&v.TS[r * TBL + c]) = pack2(b0 * __expf(gr - g2.x), b1 * __expf(gr - g2.y));
        }
    }
    wave_lds_sync();
    // (2) merge to 32 on the 16x16x16 MFMA: tmp = A_10 T_00 with lane (column l%16,
    //     rows 4 (l/16) + 0..3); then T_10^T = tmp^T (-T_11^T), the operands swapped so
    //     that lane (l%16, l/16) holds row 16 + l%16 of T0, columns 4 (l/16) + 0..3
    {
        const int c16 = l & 15, k4 = 4 * (l >> 4);
        const float4 a10 = *reinterpret_cast<const float4 *>(&M[(16 + c16) * AFL + k4]);
        const s16x4 fa = pack4(a10.x, a10.y, a10.z, a10.w);
        const s16x4 fb = pack4(M[(k4 + 0) * AFL + c16], M[(k4 + 1) * AFL + c16], M[(k4 + 2) * AFL + c16],
                               M[(k4 + 3) * AFL + c16]);
        f32x4 tmp4 = {0.f, 0.f, 0.f, 0.f};
        tmp4 = mfma16(fa, fb, tmp4);
        const float4 t11 = *reinterpret_cast<const float4 *>(&M[(16 + c16) * AFL + 16 + k4]);
        const s16x4 nt = pack4(-t11.x, -t11.y, -t11.z, -t11.w);
        const s16x4 tt = pack4(tmp4[0], tmp4[1], tmp4[2], tmp4[3]);
        f32x4 t10 = {0.f, 0.f, 0.f, 0.f};
        t10 = mfma16(tt, nt, t10);
        inv_put4<WP>(v, 16 + c16, k4, make_float4(t10[0], t10[1], t10[2], t10[3]));
    }
}

// Phase b, prep waves 0 and 2: K^T of chunk c for the next update, blocks (tokens
// 32 tb, channels 32 ib) idx = 4 q .. 4 q + 3, turned around on the MFMA (X . I) and
// stored channel-major.
template <class SM>
__device__ __forceinline__ void prep_kt(SM &sm, int b, int q, int l) {
    const int h = l >> 5, l32 = l & 31;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int idx = 4 * q + u, tb = idx >> 2, ib = idx & 3;
        f32x16 kk;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            kk = mfma(lds8(&sm.Km[b][kmo(32 * tb + l32, 4 * ib + 2 * ks + h)]), eye_b(ks, h, l32),
                      ks == 0 ? f32x16{} : kk);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            *reinterpret_cast<u32x2 *>(&sm.Kt[(32 * ib + l32) * KTL + 32 * tb + 8 * r + 4 * h]) =
                u32x2{pack2(kk[4 * r], kk[4 * r + 1]), pack2(kk[4 * r + 2], kk[4 * r + 3])};
    }
}

// Prep wave pw = 1..3, phase a: Gram block of the chunk in Km[b] on the MFMA with
// the A operand from token block am and the B operand from token block bn, so
// lane l32 holds row t = 32 bn + l32 and registers hold columns s (k_t.k_s is
// symmetric, so the diagonal blocks read either way):
//   prep wave 1: (0,0) -> A0_11 into Af (fp32), below the diagonal
//   prep wave 2: (0,1) -> H_21 into H21[b] (bf16): k_t.k_s for P, -k_t.k_s e^{g_t - g_s} for S
//   prep wave 3: (1,1) -> A0_22 into Af (fp32), below the diagonal
// with A0 = beta_t k_t.k_s.  pv[pw] holds this wave's g, beta.
template <class SM>
__device__ __forceinline__ void prep_gram(SM &sm, int b, int pw, int l) {
    const int h = l >> 5, l32 = l & 31;
    const int am = pw == 3 ? 1 : 0, bn = pw == 1 ? 0 : 1;
    const int t = 32 * bn + l32;
    const float gt = sm.pv[pw][0][t], bt = sm.pv[pw][1][t];
    float4 gqv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) gqv[q] = *reinterpret_cast<const float4 *>(&sm.pv[pw][0][32 * am + 8 * q + 4 * h]);
    // every operand read is issued before the first product, so the reads overlap
    bf16x8 fa[8], fb[8];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        fa[kb] = lds8(&sm.Km[b][kmo(32 * am + l32, 2 * kb + h)]);
        fb[kb] = lds8(&sm.Km[b][kmo(32 * bn + l32, 2 * kb + h)]);
    }
    f32x16 ga0, ga1;     // even and odd k-steps: two shorter dependent chains
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        if (kb & 1) ga1 = mfma(fa[kb], fb[kb], kb == 1 ? f32x16{} : ga1);
        else ga0 = mfma(fa[kb], fb[kb], kb == 0 ? f32x16{} : ga0);
    }
    const f32x16 gacc = ga0 + ga1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int s4 = 8 * q + 4 * h;     // column within the block
        const float4 gq4 = gqv[q];
        const float ggv[4] = {gq4.x, gq4.y, gq4.z, gq4.w};
        float a0[4];
        if (pw == 2) {
            float a1[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a0[e] = gacc[4 * q + e];
                a1[e] = -a0[e] * __expf(gt - ggv[e]);
            }
            const int o = l32 * TBL + s4;
            if (SM::kWithP)
                *reinterpret_cast<u32x2 *>(&sm.H21[b][0][o]) = u32x2{pack2(a0[0], a0[1]), pack2(a0[2], a0[3])};
            *reinterpret_cast<u32x2 *>(&sm.H21[b][SM::kS][o]) = u32x2{pack2(a1[0], a1[1]), pack2(a1[2], a1[3])};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) a0[e] = s4 + e < l32 ? bt * gacc[4 * q + e] : 0.f;
            *reinterpret_cast<float4 *>(&sm.Af[am][l32 * AFL + s4]) = make_float4(a0[0], a0[1], a0[2], a0[3]);
        }
    }
}

// ---------------------------------------------------------------- chunk streams
// The record build and the prefill forward run several (segment, head) units per
// workgroup, their chunks back to back as one stream.  The launch has G workgroups;
// workgroup j takes units j, j + G, j + 2G, ... (at most SM::kTmax of them).  At
// set-up each thread reads one unit's offsets (and slot, with records): an
// out-of-range slot raises the flag; with records, an empty unit gets the identity
// record and one with bad offsets the NaN record (written by the whole workgroup);
// without records a unit with bad offsets raises the flag and writes nothing; the
// units with tokens go into an LDS table in order.  Every wave then walks the same
// chunk stream through the table with a cursor.  The kernel's LDS layout SM provides
// units[SM::kTmax], wsum[waves], wcnt[waves][2], steps, nvalid and nspecial.

// A unit of the stream: tokens [tok, tok + n) of head `head`, record rec = slot H + head.
// At the back of the table, records written at set-up: tok = 0 identity, 1 NaN.
struct UnitEnt {
    int64_t tok, n;
    int32_t rec, head;
};

// Wave-uniform copies of values that every lane holds alike (broadcast LDS reads).
__device__ __forceinline__ int uni32(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// A position in the chunk stream: chunk c of the nc chunks of table unit q
// (q = nvalid past the end), with the unit's first token, the rows of its last
// chunk and its head copied out of the table when the cursor enters it.
struct Cursor {
    int q, c, nc, last, head;
    int64_t tok0;
};

template <class SM>
__device__ __forceinline__ void cursor_enter(const SM &sm, int nvalid, Cursor &r) {
    r.c = 0;
    if (r.q < nvalid) {
        const int64_t n = uni64(sm.units[r.q].n);
        r.tok0 = uni64(sm.units[r.q].tok);
        r.head = uni32(sm.units[r.q].head);
        r.nc = (int)((n + CH - 1) / CH);
        r.last = (int)(n - (int64_t)(r.nc - 1) * CH);
    } else {
        r.tok0 = 0;
        r.nc = r.last = r.head = 0;
    }
}

template <class SM>
__device__ __forceinline__ Cursor cursor_first(const SM &sm, int nvalid) {
    Cursor r;
    r.q = 0;
    cursor_enter(sm, nvalid, r);
    return r;
}

template <class SM>
__device__ __forceinline__ void cursor_next(const SM &sm, int nvalid, Cursor &r) {
    if (++r.c >= r.nc) {
        if (r.q < nvalid) ++r.q;
        cursor_enter(sm, nvalid, r);
    }
}

// The tokens of the cursor's chunk: first token, rows (1..CH), head.
struct StepDesc {
    int64_t tok;
    int cl, head;
};

__device__ __forceinline__ StepDesc step_desc(const Cursor &r) {
    return {r.tok0 + (int64_t)r.c * CH, r.c == r.nc - 1 ? r.last : CH, r.head};
}

// Set-up of the stream (every thread of the workgroup, NTH of them; ends with a
// workgroup barrier, after which the table, nvalid, nspecial and steps are visible).
template <class SM, int NTH>
__device__ __forceinline__ void stream_setup(SM &sm, const BuildArgs &a, bool records) {
    static_assert(SM::kTmax <= NTH, "one unit per set-up thread");
    const int th = threadIdx.x, lane = th & 63;
    const int w = __builtin_amdgcn_readfirstlane(th >> 6);
    const int64_t U = (int64_t)a.num_segments * a.H, G = gridDim.x;
    const int64_t u = (int64_t)blockIdx.x + (int64_t)th * G;
    int kind = 0;   // 0: nothing to write, 1: chunk stream, 2: identity record, 3: NaN record
    int64_t o0 = 0, o1 = 0, rec = 0;
    int hd = 0;
    if (th < SM::kTmax && u < U) {
        const int64_t seg = u / a.H;
        hd = (int)(u - seg * a.H);
        o0 = a.seg_offsets[seg];
        o1 = a.seg_offsets[seg + 1];
        const int64_t slot = records ? (int64_t)a.dst_slots[seg] : 0;
        if (records && (slot < 0 || slot >= a.num_slots)) {
            raise_flag(a.err_flag, HYPIC_EFLAG_SLOT_OUT_OF_RANGE);
        } else {
            rec = slot * a.H + hd;
            if (o0 < 0 || o1 < o0 || o1 > a.num_tokens) {
                raise_flag(a.err_flag, HYPIC_EFLAG_BAD_OFFSETS);
                kind = records ? 3 : 0;
            } else {
                kind = o1 > o0 ? 1 : (records ? 2 : 0);
            }
        }
    }
    const uint64_t mv = __ballot(kind == 1), ms = __ballot(kind >= 2);
    const uint64_t below = (1ull << lane) - 1;
    int64_t nch = kind == 1 ? (o1 - o0 + CH - 1) / CH : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) nch += __shfl_xor(nch, o);
    if (lane == 0) {
        sm.wcnt[w][0] = __popcll(mv);
        sm.wcnt[w][1] = __popcll(ms);
        sm.wsum[w] = nch;
    }
    __syncthreads();
    int pv = 0, ps = 0;
    for (int x = 0; x < w; ++x) {
        pv += sm.wcnt[x][0];
        ps += sm.wcnt[x][1];
    }
    if (kind == 1) sm.units[pv + __popcll(mv & below)] = UnitEnt{o0, o1 - o0, (int32_t)rec, hd};
    if (kind >= 2) sm.units[SM::kTmax - 1 - (ps + __popcll(ms & below))] = UnitEnt{kind - 2, 0, (int32_t)rec, hd};
    if (th == 0) {
        int nv = 0, ns = 0;
        int64_t stp = 0;
        for (int x = 0; x < NTH / 64; ++x) {
            nv += sm.wcnt[x][0];
            ns += sm.wcnt[x][1];
            stp += sm.wsum[x];
        }
        sm.nvalid = nv;
        sm.nspecial = ns;
        sm.steps = (int32_t)stp;     // a workgroup's units fit in memory: far below 2^31 chunks
    }
    __syncthreads();
}

// The records written at set-up: empty units (I, 0, ell 0) and bad offsets (NaN).
template <class SM, int NTH>
__device__ __forceinline__ void stream_special_records(const SM &sm, const BuildArgs &a) {
    const int th = threadIdx.x;
    const float nanv = __int_as_float(0x7fc00000);
    const int nspecial = uni32(sm.nspecial);
    for (int s = 0; s < nspecial; ++s) {
        const bool nanr = uni64(sm.units[SM::kTmax - 1 - s].tok) != 0;
        const int64_t r = uni32(sm.units[SM::kTmax - 1 - s].rec);
        float *P = a.pool_P + r * D * D, *S = a.pool_S + r * D * D;
        for (int x = th; x < D * D; x += NTH) {
            P[x] = nanr ? nanv : (x / D == x % D ? 1.0f : 0.0f);
            S[x] = nanr ? nanv : 0.0f;
        }
        if (th == 0) a.pool_ell[r] = nanr ? nanv : 0.0f;
    }
}

// Compute units of the current device, read once per device.
inline int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// The grid of a chunk-stream launch over U units: a multiple of the CU count (one
// resident workgroup per CU), each workgroup taking at most tmax units.
inline int64_t stream_grid(int64_t U, int tmax) {
    const int64_t cus = cu_count();
    const int64_t G = cus * ((U + cus * tmax - 1) / (cus * tmax));
    return G > U ? U : G;
}

}  // namespace
}  // namespace hypic
