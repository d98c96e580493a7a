// Segment-record build on MFMA: GDN family, d_k = d_v = 128, bf16 k/v,
// fp32 records.  bf16 MFMA operands, fp32 accumulation, fp64 ell.
//
// What it computes (besthub article "Cut First-Token Latency by 3.25x ...",
// paragraph 4; agihunt summary, "Core Approach"): the record (ell, P, S) of
// every (segment, head), T_C = e^ell P, for A_t = alpha_t (I - beta_t k_t k_t^T)
// (Gated Delta Networks, podcast companion page, reference 7).
//
// Chunked WY/UT form, chunk = 64 tokens, g = in-chunk cumulative log decay,
// G = chunk total (the plain-arithmetic statement is in build_ref.hip):
//   A0 = strictlower(beta_t k_t.k_s),   A = A0 . e^{g_t - g_s}
//   P columns X:  Y = (I + A0)^{-1} (beta . (K X));                X <- X - K^T Y
//   S columns X:  Y = (I + A )^{-1} (beta . (V - e^g . (K X)));    X <- e^G X + K^T (e^{G-g} . Y)
// The P update uses the ungated system, so no decay factor can overflow it.
// With 32-token blocks, T_ii = (I + A_ii)^{-1} and A = diag(beta) H (H: the
// block of k_t.k_s, with e^{g_t - g_s} for S, without beta),
//     Y_1 = (T_11 diag beta_1) W_1,    Y_2 = (T_22 diag beta_2) (W_2 - H_21 Y_1),
// so each system needs two 32x32 inverse factors and H_21 per chunk.
//
// Work split: one 512-thread workgroup per (segment, head), two roles.
//  * State waves 0-3 each own 32 columns of P and the same 32 columns of S
//    as eight fp32 32x32 accumulator tiles that stay in registers for the
//    whole segment (so the four waves do identical work).  Per chunk: W = K X
//    (and V - e^g . W for S), the block solve against the factors (three
//    dependent products), and the update.
//  * Prep waves 4-7 build the next chunk's factors meanwhile: the decay
//    prefix, the Gram blocks (A11, A22 in fp32, H_21 in bf16); the inverses
//    of the 32x32 diagonal blocks (4x4 forward substitution and fp32 merges
//    up to 16, one 16 -> 32 merge on the MFMA), written as T diag(beta) in
//    bf16 by each level as it finishes; prep wave 0 also loads keys and
//    values into LDS.  Prep waves 4 and 6 turn K^T around for the update in phase b.
// Two workgroup barriers per chunk: in phase a the state waves finish chunk
// c - 1 (solve, update) while the prep waves compute A of chunk c; in phase b
// the state waves form W of chunk c while the prep waves invert.
//
// Layout facts used throughout (v_mfma_f32_32x32x16_bf16): the accumulator
// and the B operand both put one column per lane, so an accumulator tile is
// the B operand of the next product after a bf16 pack (acc_to_b); the pack
// feeds contraction indices 16 half + 4h + 0..3 and 16 half + 8 + 4h + 0..3 from
// lane half h.  The rows of every state-side accumulator are kept in swizzled
// order (physical row p holds index swz(p), bits 2 and 3 swapped) so that
// those indices become 16 half + 8h + 0..7: every A operand is then one
// 16-byte LDS read from a plain row-major tile, at row swz(lane).
// X . I on the MFMA moves a token-major tile into the accumulator layout
// (one column per lane); that gives K^T and the V term of W.
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
constexpr int NT = 512;    // 4 state waves + 4 prep waves
constexpr int KML = 128;   // row length (bf16) of Km, Vm [token][channel], granules swizzled (kmo)
constexpr int KTL = 72;    // row length (bf16) of Kt [channel][token]
constexpr int AFL = 36;    // row length (fp32) of the 32x32 diagonal blocks in Af
constexpr int TBL = 40;    // row length (bf16) of the 32x32 factor tiles

struct __align__(16) Smem {
    u16 Km[2][CH * KML];       // keys, token-major, double-buffered by chunk parity
    u16 Vm[2][CH * KML];       // values, token-major, double-buffered by chunk parity
    u16 Kt[D * KTL];           // keys, channel-major
    u16 TB[2][2][2][32 * TBL]; // [chunk parity][system]: T_11 diag(beta_1), T_22 diag(beta_2) (negated for P)
    u16 H21[2][2][32 * TBL];   // [chunk parity][system]: H_21 (P), -H_21 (S), row t, column s
    float Af[2][32 * AFL];     // diagonal blocks of A0 (P system), inverted in place
    float pv[4][2][CH];        // per prep wave: g, beta of the chunk being prepared
    float inv_tmp[4][128];     // per prep wave: products inside the blocked inversion
    float egs[2][CH];          // -e^{g_t} sigma_c: the K X factor of W (S columns)
    float egrs[2][CH];         // e^{G - g_t} / sigma_{c+1}: the update factor (S columns)
    float rs[2];               // sigma_c e^G when the scale is folded back into the state, else 1
    float sig_fin;             // sigma after the last chunk
    int64_t t0, n;
    int32_t slot, state;
};

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
struct InvCtx {
    float *M, *tmp;
    u16 *TP, *TS;
    const float *bet, *gg;
};

__device__ __forceinline__ InvCtx inv_ctx(Smem &sm, int par, int blk, int pw) {
    return InvCtx{sm.Af[blk], sm.inv_tmp[pw], sm.TB[par][0][blk], sm.TB[par][1][blk], &sm.pv[pw][1][32 * blk],
                  &sm.pv[pw][0][32 * blk]};
}

// both factors of one T0 entry x at (r, c), r > c
__device__ __forceinline__ void inv_put(const InvCtx &v, int r, int c, float x) {
    const float bx = x * v.bet[c];
    v.TP[r * TBL + c] = f2bf(-bx);
    v.TS[r * TBL + c] = f2bf(bx * __expf(v.gg[r] - v.gg[c]));
}

// both factors of four consecutive T0 entries of row r, columns c .. c + 3
// (entries above the diagonal are zero in T0 and written as zero)
__device__ __forceinline__ void inv_put4(const InvCtx &v, int r, int c, float4 x) {
    const float4 b4 = *reinterpret_cast<const float4 *>(&v.bet[c]);
    const float4 g4 = *reinterpret_cast<const float4 *>(&v.gg[c]);
    const float gr = v.gg[r];
    const float b0 = x.x * b4.x, b1 = x.y * b4.y, b2 = x.z * b4.z, b3 = x.w * b4.w;
    const float e0 = r >= c ? __expf(gr - g4.x) : 0.f, e1 = r >= c + 1 ? __expf(gr - g4.y) : 0.f;
    const float e2 = r >= c + 2 ? __expf(gr - g4.z) : 0.f, e3 = r >= c + 3 ? __expf(gr - g4.w) : 0.f;
    *reinterpret_cast<u32x2 *>(&v.TP[r * TBL + c]) = u32x2{pack2(-b0, -b1), pack2(-b2, -b3)};
    *reinterpret_cast<u32x2 *>(&v.TS[r * TBL + c]) = u32x2{pack2(b0 * e0, b1 * e1), pack2(b2 * e2, b3 * e3)};
}

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
        inv_put4(v, o + i, o, x);
    }
    wave_lds_sync();
}

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
        inv_put(v, o + 4 + i, o + j, x);
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
        *reinterpret_cast<uint32_t *>(&v.TP[r * TBL + c]) = pack2(-b0, -b1);
        *reinterpret_cast<uint32_t *>(&v.TS[r * TBL + c]) = pack2(b0 * __expf(gr - g2.x), b1 * __expf(gr - g2.y));
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
        inv_put4(v, 16 + c16, k4, make_float4(t10[0], t10[1], t10[2], t10[3]));
    }
}

// Phase b, prep waves 0 and 2: K^T of chunk c for the next update, blocks (tokens
// 32 tb, channels 32 ib) idx = 4 q .. 4 q + 3, turned around on the MFMA (X . I) and
// stored channel-major.
__device__ __forceinline__ void prep_kt(Smem &sm, int b, int q, int l) {
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
__device__ __forceinline__ void prep_gram(Smem &sm, int b, int pw, int l) {
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
            *reinterpret_cast<u32x2 *>(&sm.H21[b][0][o]) = u32x2{pack2(a0[0], a0[1]), pack2(a0[2], a0[3])};
            *reinterpret_cast<u32x2 *>(&sm.H21[b][1][o]) = u32x2{pack2(a1[0], a1[1]), pack2(a1[2], a1[3])};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) a0[e] = s4 + e < l32 ? bt * gacc[4 * q + e] : 0.f;
            *reinterpret_cast<float4 *>(&sm.Af[am][l32 * AFL + s4]) = make_float4(a0[0], a0[1], a0[2], a0[3]);
        }
    }
}

__global__ __launch_bounds__(NT, 1) void gdn_build_mfma_kernel(BuildArgs a) {
    __shared__ Smem sm;

    const int th = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(th >> 6);
    const int head = blockIdx.x % a.H;
    const int seg = blockIdx.x / a.H;

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
    // the upper triangles of the T diag(beta) tiles stay zero for the whole segment
    for (int e = th; e < (int)(sizeof(sm.TB) / 16); e += NT) reinterpret_cast<u32x4 *>(&sm.TB[0][0][0][0])[e] = u32x4{};
    __syncthreads();
    const int state = sm.state;
    if (state == 1) return;
    const int64_t t0 = sm.t0;
    const int64_t n = state == 2 ? 0 : sm.n;
    const int64_t slot = sm.slot;
    const int64_t nc = (n + CH - 1) / CH;
    const float nanv = __int_as_float(0x7fc00000);
    const bool bad = state == 2;
    const int64_t rec = slot * a.H + head;

    if (w < 4) {
        // =============================== state waves ===============================
        // column block 0: P columns 32w .. 32w + 31; column block 1: the same S columns
        const int col = 32 * w;
        f32x16 st[2][4];                          // [column block][row block], rows swizzled
        bf16x8 wb[2][2][2];                       // W of the chunk in flight as B operands [cb][tb][half]
        {
            const int h = (th & 63) >> 5, l32 = th & 31;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        st[cb][mb][r] = (cb == 0 && swz(32 * mb + acc_row(r, h)) == col + l32) ? 1.0f : 0.0f;
        }
        __syncthreads();                                            // prologue: chunk 0 staged
        for (int64_t i = 0; i <= nc; ++i) {
            int thv = th;
            asm volatile("" : "+v"(thv));
            const int h = (thv & 63) >> 5, l32 = thv & 31;
            // ---- phase a: solve and update of chunk i - 1
            if (i >= 1) {
                const int b = (int)((i - 1) & 1);
                const int rr = swz(l32) * TBL + 8 * h;
                {
                    const float rsc = sm.rs[b];
                    if (rsc != 1.0f) {
                        // the pending decay sigma_c e^G is folded into the S state (rare)
#pragma unroll
                        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                            for (int r = 0; r < 16; ++r) st[1][mb][r] *= rsc;
                    }
                }
                // factor operands [system][k-step]: T_11 diag b_1 and H_21 read up front
                bf16x8 f0[2][2], fh[2][2], f1[2][2];
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        f0[cb][half] = lds8(&sm.TB[b][cb][0][rr + 16 * half]);
                        fh[cb][half] = lds8(&sm.H21[b][cb][rr + 16 * half]);
                    }
                f32x16 y1[2], y2[2];     // [column block = system]
                bf16x8 yb[4][2];         // B operands of the update, [k-step][system]
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    y1[cb] = mfma(f0[cb][0], wb[cb][0][0], f32x16{});
                    y1[cb] = mfma(f0[cb][1], wb[cb][0][1], y1[cb]);
                }
                // W_2 - H_21 Y_1 (H21 carries the sign that makes this a sum for both
                // systems; P's factors and Y are negated), accumulated onto W_2 itself: a
                // B operand pack holds the registers of its accumulator in order
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const f32x8 w0 = __builtin_convertvector(wb[cb][1][0], f32x8);
                    const f32x8 w1 = __builtin_convertvector(wb[cb][1][1], f32x8);
                    y2[cb] = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
                    yb[0][cb] = acc_to_b(y1[cb], 0);
                    yb[1][cb] = acc_to_b(y1[cb], 1);
                    y2[cb] = mfma(fh[cb][0], yb[0][cb], y2[cb]);
                    y2[cb] = mfma(fh[cb][1], yb[1][cb], y2[cb]);
                }
                // S: Y_1 times e^{G - g} / sigma for the update
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 e0 = tok4(sm.egrs[b], 0, q, h);
                    y1[1][4 * q] *= e0.x; y1[1][4 * q + 1] *= e0.y;
                    y1[1][4 * q + 2] *= e0.z; y1[1][4 * q + 3] *= e0.w;
                }
                yb[0][1] = acc_to_b(y1[1], 0);
                yb[1][1] = acc_to_b(y1[1], 1);
                // T_22 diag b_2, read while the first half of the update runs
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int half = 0; half < 2; ++half) f1[cb][half] = lds8(&sm.TB[b][cb][1][rr + 16 * half]);
                // X += K^T Y (the P factors are stored negated): A operand = Kt rows (channels)
                // swz(32 mb + lane); token steps 0, 1 need only Y_1, so they overlap the
                // Y_2 chain below
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    bf16x8 kt[4];
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb) kt[mb] = lds8(&sm.Kt[swz(32 * mb + l32) * KTL + 16 * s2 + 8 * h]);
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                        for (int cb = 0; cb < 2; ++cb) st[cb][mb] = mfma(kt[mb], yb[s2][cb], st[cb][mb]);
                }
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const bf16x8 u0 = acc_to_b(y2[cb], 0), u1 = acc_to_b(y2[cb], 1);
                    y2[cb] = mfma(f1[cb][0], u0, f32x16{});
                    y2[cb] = mfma(f1[cb][1], u1, y2[cb]);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 e1 = tok4(sm.egrs[b], 1, q, h);
                    y2[1][4 * q] *= e1.x; y2[1][4 * q + 1] *= e1.y;
                    y2[1][4 * q + 2] *= e1.z; y2[1][4 * q + 3] *= e1.w;
                }
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    yb[2][cb] = acc_to_b(y2[cb], 0);
                    yb[3][cb] = acc_to_b(y2[cb], 1);
                }
#pragma unroll
                for (int s2 = 2; s2 < 4; ++s2) {
                    bf16x8 kt[4];
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb) kt[mb] = lds8(&sm.Kt[swz(32 * mb + l32) * KTL + 16 * s2 + 8 * h]);
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                        for (int cb = 0; cb < 2; ++cb) st[cb][mb] = mfma(kt[mb], yb[s2][cb], st[cb][mb]);
                }
            }
            lds_barrier();                                          // a -> b
            // ---- phase b: W of chunk i
            if (i < nc) {
                const int b = (int)(i & 1);
                f32x16 z[2][2];                   // [column block][token block], rows swizzled
                // K X: A operand = Km rows (tokens) swz(32 mb + lane), B = state rows in swizzled order
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) {
                    bf16x8 sb[2];
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb) sb[cb] = acc_to_b(st[cb][kb >> 1], kb & 1);
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb) {
                        const bf16x8 km = lds8(&sm.Km[b][kmo(swz(32 * mb + l32), 2 * kb + h)]);
#pragma unroll
                        for (int cb = 0; cb < 2; ++cb)
                            z[cb][mb] = mfma(km, sb[cb], kb == 0 ? f32x16{} : z[cb][mb]);
                    }
                }
                {
                    // S block: W = V - e^g . (K X): scale, then add V turned around on the MFMA
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const float4 e4 = tok4(sm.egs[b], mb, q, h);
                            z[1][mb][4 * q] *= e4.x; z[1][mb][4 * q + 1] *= e4.y;
                            z[1][mb][4 * q + 2] *= e4.z; z[1][mb][4 * q + 3] *= e4.w;
                        }
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const bf16x8 eye = eye_b(ks, h, l32);
#pragma unroll
                        for (int mb = 0; mb < 2; ++mb)
                            z[1][mb] = mfma(lds8(&sm.Vm[b][kmo(swz(32 * mb + l32), 4 * w + 2 * ks + h)]), eye, z[1][mb]);
                    }
                }
                // kept across the barrier as bf16 B operands: half the registers of W
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                        for (int half = 0; half < 2; ++half) wb[cb][mb][half] = acc_to_b(z[cb][mb], half);
            }
            __syncthreads();                                        // b -> next a
        }
        // ---- record: physical row p of a tile holds channel swz(p); S = sigma X
        const int h = (th & 63) >> 5, l32 = th & 31;
        const float sfin = sm.sig_fin;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            float *dst = (cb == 0 ? a.pool_P : a.pool_S) + rec * D * D;
            const float sc = cb == 0 ? 1.0f : sfin;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    dst[(int64_t)swz(32 * mb + acc_row(r, h)) * D + col + l32] = bad ? nanv : st[cb][mb][r] * sc;
        }
    } else {
        // =============================== prep waves ===============================
        // Their work is a chain of short dependent steps that shares each SIMD with a
        // state wave's long MFMA stream: issue priority keeps the chain moving.
        __builtin_amdgcn_s_setprio(3);
        const int pw = w - 4;
        const int pl = th & 63;
        // every prep wave loads la and beta of a chunk itself (lane = token)
        const float *bq = a.beta ? a.beta + (t0 + pl) * a.b_st + head * a.b_sh : nullptr;
        const float *lq = a.log_alpha ? a.log_alpha + (t0 + pl) * a.la_st + head * a.la_sh : nullptr;
        float lar = 0.f, br = 0.f;
#define HYPIC_FETCH_G(BASE)                                                                          \
    do {                                                                                             \
        const int64_t base_ = (BASE), rem_ = n - base_;                                              \
        const int cl_ = rem_ < CH ? (int)rem_ : CH;                                                  \
        br = pl < cl_ ? (bq ? bq[base_ * a.b_st] : 1.0f) : 0.0f;                                     \
        lar = (pl < cl_ && lq) ? lq[base_ * a.la_st] : 0.0f;                                         \
    } while (0)
        if (nc > 0) HYPIC_FETCH_G(0);
        if (pw == 0) {
            // ---- prep wave 0: loads keys and values, the decay factors, ell; inverts
            //      block 0 of the P system.
            // Keys and values go straight from HBM into Km/Vm (global_load_lds): the
            // instruction for rows 4u .. 4u + 3 lands lane l's 16 bytes in row 4u + l / 16,
            // slot l % 16, so the lane loads the granule that kmo puts there.  Rows past
            // the segment repeat its last row (finite values; their beta is zero).
            const u16 *kh = static_cast<const u16 *>(a.k) + t0 * a.k_st + head * a.k_sh;
            const u16 *vh = static_cast<const u16 *>(a.v) + t0 * a.v_st + head * a.v_sh;
            // full chunks (the common case): element offsets of this lane's sixteen
            // pieces, relative to the chunk's first row, fixed for the whole segment
            const bool small_st = (int64_t)CH * (a.k_st > a.v_st ? a.k_st : a.v_st) < (1LL << 30);
            uint32_t ko[16], vo[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int t = 4 * u + (pl >> 4), g = (pl & 15) ^ (t & 15);
                ko[u] = small_st ? (uint32_t)(t * a.k_st + 8 * g) : 0u;
                vo[u] = small_st ? (uint32_t)(t * a.v_st + 8 * g) : 0u;
            }
#define HYPIC_LOAD_KV(BASE, BUF)                                                                     \
    do {                                                                                             \
        const int64_t base_ = (BASE), rem_ = n - base_;                                              \
        const u16 *kc_ = kh + base_ * a.k_st, *vc_ = vh + base_ * a.v_st;                            \
        if (rem_ >= CH && small_st) {                                                                \
            _Pragma("unroll") for (int u_ = 0; u_ < 16; ++u_) {                                      \
                __builtin_amdgcn_global_load_lds(kc_ + ko[u_], &sm.Km[BUF][4 * u_ * KML], 16, 0, 0);  \
                __builtin_amdgcn_global_load_lds(vc_ + vo[u_], &sm.Vm[BUF][4 * u_ * KML], 16, 0, 0);  \
            }                                                                                        \
        } else {                                                                                     \
            const int cl_ = rem_ < CH ? (int)rem_ : CH;                                              \
            int l_ = pl;                                                                             \
            asm volatile("" : "+v"(l_));                                                             \
            const int r_ = l_ >> 4, p_ = l_ & 15;                                                    \
            _Pragma("unroll") for (int u_ = 0; u_ < 16; ++u_) {                                      \
                const int t_ = 4 * u_ + r_, ts_ = t_ < cl_ ? t_ : cl_ - 1;                           \
                const int g_ = p_ ^ (t_ & 15);                                                       \
                __builtin_amdgcn_global_load_lds(kc_ + ts_ * a.k_st + 8 * g_,                        \
                                                 &sm.Km[BUF][4 * u_ * KML], 16, 0, 0);               \
                __builtin_amdgcn_global_load_lds(vc_ + ts_ * a.v_st + 8 * g_,                        \
                                                 &sm.Vm[BUF][4 * u_ * KML], 16, 0, 0);               \
            }                                                                                        \
        }                                                                                            \
    } while (0)
            double ell = 0.0;     // this lane's tokens; summed over the wave at the end
            // S = sigma X for the S columns: the decay e^G of each chunk is carried in
            // sigma and folded into X only when sigma would drop below 2^-60, so the
            // state waves do not rescale X every chunk.
            float sig = 1.0f;
            if (pl == 0) sm.sig_fin = 1.0f;
            if (nc > 0) {
                HYPIC_LOAD_KV(0, 0);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            __syncthreads();                                        // prologue: chunk 0 staged
            for (int64_t i = 0; i <= nc; ++i) {
                int thv = th;
                asm volatile("" : "+v"(thv));
                const int l = thv & 63;
                // ---- phase a: decay factors of chunk i; keys and values of chunk i + 1 start
                if (i < nc) {
                    const int b = (int)(i & 1);
                    const float la_i = lar, b_i = br;
                    if (i + 1 < nc) HYPIC_LOAD_KV((i + 1) * CH, b ^ 1);     // lands during this chunk
                    const float gv = wave_prefix_sum(la_i);
                    sm.pv[0][0][l] = gv;
                    sm.pv[0][1][l] = b_i;
                    const float gt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), 63));
                    const float sp = sig * __expf(gt);
                    const bool fold = sp < 0x1p-60f;
                    const float inv = fold ? 1.0f : 1.0f / sp;
                    sm.egs[b][l] = -__expf(gv) * sig;
                    sm.egrs[b][l] = __expf(gt - gv) * inv;
                    if (l == 63) {
                        sm.rs[b] = fold ? sp : 1.0f;
                        sm.sig_fin = fold ? 1.0f : sp;
                    }
                    sig = fold ? 1.0f : sp;
                    ell += (double)la_i;
                }
                lds_barrier();                                      // a -> b
                // ---- phase b: keys and values of chunk i + 1 land in the other buffers;
                //      gates of chunk i + 1 (read in phase b, so that their wait falls at
                //      its end); factors of block 0 of the P system
                if (i + 1 < nc) HYPIC_FETCH_G((i + 1) * CH);
                if (i < nc) prep_kt(sm, (int)(i & 1), 0, l);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // chunk i + 1 has landed
                __syncthreads();                                    // b -> next a
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) ell += __shfl_xor(ell, o);
            if (th == 256) a.pool_ell[rec] = bad ? nanv : (float)ell;
#undef HYPIC_LOAD_KV
        } else {
            // ---- prep waves 1-3: Gram block and A in phase a; one factor block in phase b
            __syncthreads();                                        // prologue: chunk 0 staged
            for (int64_t i = 0; i <= nc; ++i) {
                int thv = th;
                asm volatile("" : "+v"(thv));
                const int l = thv & 63;
                if (i < nc) {
                    const int b = (int)(i & 1);
                    const float la_i = lar, b_i = br;
                    sm.pv[pw][0][l] = wave_prefix_sum(la_i);
                    sm.pv[pw][1][l] = b_i;
                    wave_lds_sync();
                    prep_gram(sm, b, pw, l);
                    if (pw != 2) {
                        wave_lds_sync();
                        prep_invert1(inv_ctx(sm, b, pw >> 1, pw), l);
                    }
                }
                lds_barrier();                                      // a -> b
                if (i + 1 < nc) HYPIC_FETCH_G((i + 1) * CH);        // gates of chunk i + 1
                if (i < nc && pw != 2) prep_invert2(inv_ctx(sm, (int)(i & 1), pw >> 1, pw), l);
                if (i < nc && pw == 2) prep_kt(sm, (int)(i & 1), 1, l);
                __syncthreads();                                    // b -> next a
            }
        }
#undef HYPIC_FETCH_G
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_build_mfma(const BuildArgs &a, hipStream_t stream, bool *taken) {
    *taken = false;
    if (a.family != HYPIC_GDN || a.kv_dtype != HYPIC_BF16 || a.dk != 128 || a.dv != 128) return hipSuccess;
    if (!aligned16(a.k) || !aligned16(a.v) || (a.k_st % 8) || (a.k_sh % 8) || (a.v_st % 8) || (a.v_sh % 8))
        return hipSuccess;
    *taken = true;
    const dim3 grid((unsigned)((int64_t)a.num_segments * a.H));
    hipLaunchKernelGGL(gdn_build_mfma_kernel, grid, dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace hypic
