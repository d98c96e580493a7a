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
//
// The triangular systems are solved on each wave's own columns instead of
// forming the 64x64 inverse.  With 32-row blocks,
//     Y_1 = T_11 R_1,   Y_2 = T_22 (R_2 - A_21 Y_1),   T_ii = (I + A_ii)^{-1},
// so the shared work is the two 32x32 diagonal inverses of each system (16x16
// diagonal blocks by forward substitution, one 16 -> 32 merge in fp32); the
// rest is six MFMAs per wave.
//
// Work split: one 512-thread workgroup (8 waves) per (segment, head).  Wave w
// owns 32 columns of [P | S] (waves 0-3: P, waves 4-7: S) as four fp32 32x32
// accumulator tiles that stay in registers for the whole segment.  The 32x32
// accumulator layout and the B-operand layout of v_mfma_f32_32x32x16_bf16 both
// put one column per lane, so an accumulator tile becomes the B operand of the
// next product after a bf16 pack; only the order of the contraction index
// changes, and the A operand is read in that same order.  The same fact moves
// token-major tiles into the accumulator layout: X . I on the MFMA returns X
// with one column per lane, which gives K^T for the update's A operand and V
// in the layout of K X.
#include "hypic_internal.h"

namespace hypic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

constexpr int CH = 64;     // tokens per chunk
constexpr int D = 128;     // d_k = d_v
constexpr int NT = 512;    // 8 waves
constexpr int KTL = 72;    // row length (bf16) of Kt [channel][token]
constexpr int KML = 136;   // row length (bf16) of Km, Vm [token][channel]
constexpr int AFL = 68;    // row length (fp32) of A0 and A
constexpr int TBL = 72;    // row length (bf16) of the bf16 copies of T0 and T

// Kt (tokens), Km (channels) and TB (columns) are stored with the index
// swizzle below, so that every MFMA A operand in acc_to_b order is one
// 16-byte LDS read.
struct __align__(16) Smem {
    u16 Kt[D * KTL];           // keys, channel-major: A operand of the update
    u16 Km[CH * KML];          // keys, token-major: Gram, K X, turn-around
    u16 Vm[CH * KML];          // values, token-major, plain order
    float A0[CH * AFL];        // A0; its 32x32 diagonal blocks become T0_11, T0_22
    float A1[CH * AFL];        // A;  its 32x32 diagonal blocks become T_11,  T_22
    u16 TB[2][CH * TBL];       // bf16 [T_11 0; -A_21 T_22] of both systems (the solve's A operands)
    float scratch[2][512];     // 16 -> 32 merge temporaries
    float g[CH], eg[CH], egr[CH], beta[CH], la[CH];
    float eG;
    int64_t t0, n;
    int32_t slot, state;
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(u16, x) | ((uint32_t)__builtin_bit_cast(u16, y) << 16);
}

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                        float a7) {
    u32x4 u = {pack2(a0, a1), pack2(a2, a3), pack2(a4, a5), pack2(a6, a7)};
    return __builtin_bit_cast(bf16x8, u);
}

// 8 consecutive bf16 from LDS (16-byte aligned)
__device__ __forceinline__ bf16x8 lds8(const u16 *p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}

// Row of the 32x32 accumulator element held in register r by lane half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// B operand (k-step `half` of a 32-row block) from accumulator registers: element e
// of the fragment is accumulator row 16 half + 4h + e for e < 4, 16 half + 8 + 4h + e - 4 after.
__device__ __forceinline__ bf16x8 acc_to_b(const f32x16 &c, int half) {
    const int o = 8 * half;
    return pack8(c[o + 0], c[o + 1], c[o + 2], c[o + 3], c[o + 4], c[o + 5], c[o + 6], c[o + 7]);
}

// Storage position of index c: bits 2 and 3 swapped (an involution inside each
// group of 16).  The eight indices that lane half h contributes in acc_to_b
// order, 16 half + 4h + 0..3 and 16 half + 8 + 4h + 0..3, then sit at
// 16 half + 8h + 0..7.
__device__ __forceinline__ int swz(int c) { return (c & ~12) | ((c & 4) << 1) | ((c & 8) >> 1); }

// B operand of the identity for k-step ks: column l32; row 16 ks + 8h + e of the
// operand holds index c of the block, with c = swz(16 ks + 8h + e) when the A
// operand is stored swizzled, else c = 16 ks + 8h + e.
__device__ __forceinline__ bf16x8 eye_b(int ks, int h, int l32, bool swizzled) {
    bf16x8 e8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int p = 16 * ks + 8 * h + e;
        e8[e] = (__bf16)(((swizzled ? swz(p) : p) == l32) ? 1.0f : 0.0f);
    }
    return e8;
}

// 4 per-row values of accumulator rows 32 mb + 8 q + 4h + 0..3 (registers 4q..4q+3)
__device__ __forceinline__ float4 rows4(const float *v, int mb, int q, int h) {
    return *reinterpret_cast<const float4 *>(v + 32 * mb + 8 * q + 4 * h);
}

__device__ __forceinline__ u16 f2bf(float x) { return __builtin_bit_cast(u16, (__bf16)x); }

__global__ __launch_bounds__(NT, 1) void gdn_build_mfma_kernel(BuildArgs a) {
    __shared__ Smem sm;

    const int th = threadIdx.x;
    const int w = th >> 6;
    const int head = blockIdx.x % a.H;
    const int seg = blockIdx.x / a.H;
    const bool isS = w >= 4;
    const int col0 = 32 * (w & 3);           // first column of this wave's slab (within P or S)

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
    __syncthreads();
    const int state = sm.state;
    if (state == 1) return;
    const int64_t t0 = sm.t0;
    const int64_t n = state == 2 ? 0 : sm.n;
    const int64_t slot = sm.slot;

    // state slab: P = I, S = 0
    f32x16 st[4];
    {
        const int h = (th & 63) >> 5, l32 = th & 31;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                st[mb][r] = (!isS && 32 * mb + acc_row(r, h) == col0 + l32) ? 1.0f : 0.0f;
    }
    double ell = 0.0;   // thread 256 (wave 4, lane 0)
    // upper-right 16x16 blocks of T_11 and T_22 (zero, never written again)
    for (int e = th; e < 2 * 2 * 16 * 16; e += NT) {
        const int m = e >> 9, b = (e >> 8) & 1, i = (e >> 4) & 15, j = e & 15;
        sm.TB[m][(32 * b + i) * TBL + 32 * b + 16 + j] = 0;
    }

    const u16 *kp = static_cast<const u16 *>(a.k);
    const u16 *vp = static_cast<const u16 *>(a.v);
    // per thread: token row th / 8, 16 channels from 16 (th % 8): two 16-byte pieces of k and of v
    uint4 kreg[2], vreg[2];
    float breg = 0.f, lareg = 0.f;

    auto fetch = [&](int64_t base) {
        int thf = th;
        asm volatile("" : "+v"(thf));
        const int lt = thf >> 3, lc = 16 * (thf & 7);
        const int64_t rem = n - base;
        const int cl = rem < CH ? (int)rem : CH;
        const int64_t t = t0 + base + lt;
        if (lt < cl) {
            const uint4 *ks = reinterpret_cast<const uint4 *>(kp + t * a.k_st + head * a.k_sh + lc);
            const uint4 *vs = reinterpret_cast<const uint4 *>(vp + t * a.v_st + head * a.v_sh + lc);
            kreg[0] = ks[0]; kreg[1] = ks[1];
            vreg[0] = vs[0]; vreg[1] = vs[1];
        } else {
            kreg[0] = kreg[1] = vreg[0] = vreg[1] = make_uint4(0, 0, 0, 0);
        }
        if (th < CH) {
            const int64_t tt = t0 + base + th;
            breg = th < cl ? (a.beta ? a.beta[tt * a.b_st + head * a.b_sh] : 1.0f) : 0.0f;
            lareg = (th < cl && a.log_alpha) ? a.log_alpha[tt * a.la_st + head * a.la_sh] : 0.0f;
        }
    };

    if (n > 0) fetch(0);

    for (int64_t base = 0; base < n; base += CH) {
        // Lane indices re-derived from an opaque copy each chunk: otherwise the
        // compiler hoists every lane-dependent LDS address out of the loop and
        // runs out of registers holding them.
        int thv = th;
        asm volatile("" : "+v"(thv));
        const int l = thv & 63, h = l >> 5, l32 = l & 31;
        const int lt = thv >> 3, lc = 16 * (thv & 7);

        // ---------------- 1. stage keys, values (token-major) and gates
        *reinterpret_cast<uint4 *>(&sm.Km[lt * KML + lc]) = make_uint4(kreg[0].x, kreg[0].y, kreg[1].x, kreg[1].y);
        *reinterpret_cast<uint4 *>(&sm.Km[lt * KML + lc + 8]) =
            make_uint4(kreg[0].z, kreg[0].w, kreg[1].z, kreg[1].w);
        *reinterpret_cast<uint4 *>(&sm.Vm[lt * KML + lc]) = vreg[0];
        *reinterpret_cast<uint4 *>(&sm.Vm[lt * KML + lc + 8]) = vreg[1];
        if (thv < CH) { sm.la[thv] = lareg; sm.beta[thv] = breg; }
        if (base + CH < n) fetch(base + CH);     // next chunk's loads fly during this chunk
        __syncthreads();                                                   // B1

        // ---------------- 2. decay prefix (wave 0) | ell (wave 4) | Gram blocks (waves 1-3)
        //                     | K^T by turn-around (all) | Z = K X on own columns (all)
        f32x16 gacc;
        const int gmb = (w >= 2) ? 1 : 0, gnb = (w == 3) ? 1 : 0;
        if (w == 0) {
            // lane t: g_t = sum_{s<=t} log alpha_s (inclusive scan), G = g_63
            float gv = sm.la[l];
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(gv, o);
                if (l >= o) gv += y;
            }
            const float gt = __shfl(gv, 63);
            sm.g[l] = gv;
            sm.eg[l] = __expf(gv);
            sm.egr[l] = __expf(gt - gv);
            if (l == 63) sm.eG = __expf(gt);
        } else if (w == 4) {
            // the chunk total of log alpha in fp64, accumulated by thread 256
            double gd = (double)sm.la[l];
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) gd += __shfl_xor(gd, o);
            ell += gd;
        } else if (w <= 3) {
#pragma unroll
            for (int r = 0; r < 16; ++r) gacc[r] = 0.f;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const bf16x8 fa = lds8(&sm.Km[(32 * gmb + l32) * KML + 16 * kb + 8 * h]);
                const bf16x8 fb = gmb == gnb ? fa : lds8(&sm.Km[(32 * gnb + l32) * KML + 16 * kb + 8 * h]);
                gacc = mfma(fa, fb, gacc);
            }
        }
        {
            // wave w writes K^T of the 32x32 block (tokens 32 tb.., channels 32 ib..)
            const int tb = w >> 2, ib = w & 3;
            f32x16 kk;
#pragma unroll
            for (int r = 0; r < 16; ++r) kk[r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                kk = mfma(lds8(&sm.Km[(32 * tb + l32) * KML + 32 * ib + 16 * ks + 8 * h]), eye_b(ks, h, l32, true),
                          kk);
            // registers 4q..4q+3: tokens 8q + 4h + 0..3 of the block, stored at their swizzled positions
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x2 v2 = {pack2(kk[4 * q], kk[4 * q + 1]), pack2(kk[4 * q + 2], kk[4 * q + 3])};
                *reinterpret_cast<u32x2 *>(
                    &sm.Kt[(32 * ib + l32) * KTL + 32 * tb + 16 * (q >> 1) + 8 * h + 4 * (q & 1)]) = v2;
            }
        }
        f32x16 z[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) z[mb][r] = 0.f;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            const bf16x8 sb = acc_to_b(st[kb >> 1], kb & 1);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                z[mb] = mfma(lds8(&sm.Km[(32 * mb + l32) * KML + 16 * kb + 8 * h]), sb, z[mb]);
            }
        }
        __syncthreads();                                                   // B2

        // ---------------- 3. A0, A (waves 1-3) | right-hand sides R on own columns (all)
        if (w >= 1 && w <= 3) {
            const int s = 32 * gnb + l32;
            const float gs = sm.g[s];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 b4 = rows4(sm.beta, gmb, q, h), g4 = rows4(sm.g, gmb, q, h);
                const float bq[4] = {b4.x, b4.y, b4.z, b4.w}, gq[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 32 * gmb + 8 * q + 4 * h + e;
                    float a0 = 0.f, a1 = 0.f;
                    if (s < t) {
                        a0 = bq[e] * gacc[4 * q + e];
                        a1 = a0 * __expf(gq[e] - gs);
                    }
                    sm.A0[t * AFL + s] = a0;
                    sm.A1[t * AFL + s] = a1;
                    if (w == 2) {          // block (1,0): A_21, negated, into the bf16 copies
                        sm.TB[0][t * TBL + swz(s)] = f2bf(-a0);
                        sm.TB[1][t * TBL + swz(s)] = f2bf(-a1);
                    }
                }
            }
        }
        if (isS) {
            // R = beta (V - e^g Z): scale, then add V turned around on the MFMA
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 e4 = rows4(sm.eg, mb, q, h);
                    z[mb][4 * q] *= -e4.x; z[mb][4 * q + 1] *= -e4.y;
                    z[mb][4 * q + 2] *= -e4.z; z[mb][4 * q + 3] *= -e4.w;
                }
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    z[mb] = mfma(lds8(&sm.Vm[(32 * mb + l32) * KML + col0 + 16 * ks + 8 * h]),
                                 eye_b(ks, h, l32, false), z[mb]);
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 b4 = rows4(sm.beta, mb, q, h);
                z[mb][4 * q] *= b4.x; z[mb][4 * q + 1] *= b4.y;
                z[mb][4 * q + 2] *= b4.z; z[mb][4 * q + 3] *= b4.w;
            }
        __syncthreads();                                                   // B3

        // ---------------- 4. 16x16 diagonal blocks by forward substitution: wave 0 -> T0, wave 1 -> T
        if (w <= 1) {
            float *M = w == 0 ? sm.A0 : sm.A1;
            const int R = 16 * (l >> 4), j = l & 15;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = 0.f;
#pragma unroll
                for (int s = 0; s < i; ++s) acc += M[(R + i) * AFL + R + s] * x[s];
                x[i] = (i == j) ? 1.0f : (i < j ? 0.0f : -acc);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                M[(R + i) * AFL + R + j] = x[i];
                sm.TB[w][(R + i) * TBL + R + swz(j)] = f2bf(x[i]);
            }
        }
        __syncthreads();                                                   // B4

        // ---------------- 5. 16 -> 32: T_10 = -T_11 A_10 T_00 in each 32x32 diagonal block of
        //                     both systems, one (system, block) per wave 0-3
        const int mrow = 4 * (l >> 4), mcol = l & 15;
        if (w < 4) {
            const float *M = (w >> 1) ? sm.A1 : sm.A0;
            const int R0 = 32 * (w & 1), R1 = R0 + 16;
            float tl[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) tl[k] = M[(R0 + k) * AFL + R0 + mcol];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int k = 0; k < 16; ++k) acc += M[(R1 + mrow + r) * AFL + R0 + k] * tl[k];
                sm.scratch[w >> 1][256 * (w & 1) + (mrow + r) * 16 + mcol] = acc;
            }
        }
        __syncthreads();                                                   // B5
        if (w < 4) {
            const int mat = w >> 1;
            float *M = mat ? sm.A1 : sm.A0;
            const int R0 = 32 * (w & 1), R1 = R0 + 16;
            float tc[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) tc[k] = sm.scratch[mat][256 * (w & 1) + k * 16 + mcol];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int k = 0; k < 16; ++k) acc += M[(R1 + mrow + r) * AFL + R1 + k] * tc[k];
                M[(R1 + mrow + r) * AFL + R0 + mcol] = -acc;
                sm.TB[mat][(R1 + mrow + r) * TBL + R0 + swz(mcol)] = f2bf(-acc);
            }
        }
        __syncthreads();                                                   // B6

        // ---------------- 6. solve on own columns, then the carry update
        {
            const u16 *M = sm.TB[isS ? 1 : 0];
            f32x16 y0, y2;
#pragma unroll
            for (int r = 0; r < 16; ++r) { y0[r] = 0.f; y2[r] = 0.f; }
#pragma unroll
            for (int half = 0; half < 2; ++half)                                       // Y_1 = T_11 R_1
                y0 = mfma(lds8(&M[l32 * TBL + 16 * half + 8 * h]), acc_to_b(z[0], half), y0);
#pragma unroll
            for (int half = 0; half < 2; ++half)                                       // R_2 - A_21 Y_1
                z[1] = mfma(lds8(&M[(32 + l32) * TBL + 16 * half + 8 * h]), acc_to_b(y0, half), z[1]);
#pragma unroll
            for (int half = 0; half < 2; ++half)                                       // Y_2 = T_22 (..)
                y2 = mfma(lds8(&M[(32 + l32) * TBL + 32 + 16 * half + 8 * h]), acc_to_b(z[1], half), y2);
            if (isS) {
                // S: e^G X + K^T (e^{G-g} . Y)
                const float eG = sm.eG;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 e0 = rows4(sm.egr, 0, q, h), e1 = rows4(sm.egr, 1, q, h);
                    y0[4 * q] *= e0.x; y0[4 * q + 1] *= e0.y; y0[4 * q + 2] *= e0.z; y0[4 * q + 3] *= e0.w;
                    y2[4 * q] *= e1.x; y2[4 * q + 1] *= e1.y; y2[4 * q + 2] *= e1.z; y2[4 * q + 3] *= e1.w;
                }
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) st[mb][r] *= eG;
            } else {
                // P: X - K^T Y
#pragma unroll
                for (int r = 0; r < 16; ++r) { y0[r] = -y0[r]; y2[r] = -y2[r]; }
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 yb = acc_to_b(s < 2 ? y0 : y2, s & 1);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    st[mb] = mfma(lds8(&sm.Kt[(32 * mb + l32) * KTL + 16 * s + 8 * h]), yb, st[mb]);
                }
            }
        }
        __syncthreads();                                                   // B7
    }

    // ---------------- record
    const int h = (th & 63) >> 5, l32 = th & 31;
    const float nanv = __int_as_float(0x7fc00000);
    const bool bad = state == 2;
    const int64_t rec = slot * a.H + head;
    float *dst = isS ? a.pool_S + rec * D * D : a.pool_P + rec * D * D;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dst[(int64_t)(32 * mb + acc_row(r, h)) * D + col0 + l32] = bad ? nanv : st[mb][r];
    if (th == 256) a.pool_ell[rec] = bad ? nanv : (float)ell;
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
