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
//   M    = K K^T                                  Gram, MFMA
//   A0   = strictlower(beta_t M),  A = A0 . e^{g_t - g_s}
//   T0   = (I + A0)^{-1},  T = (I + A)^{-1}       16x16 diagonal blocks by
//                                                  substitution, then block merges
//   W0   = T0 diag(beta) K,  Ws = T diag(beta e^g) K,  U = T diag(beta) V   (MFMA)
//   P   <- P - K^T (W0 P)                                              (MFMA)
//   S   <- e^G S + K^T diag(e^{G-g}) (U - Ws S)                        (MFMA)
// The P update uses the ungated system (no decay factor can overflow it).
//
// Work split: one 512-thread workgroup (8 waves) per (segment, head).  Wave w
// owns 32 columns of [P | S] (waves 0-3: P, waves 4-7: S) as 4 fp32 32x32
// accumulator tiles that stay in registers for the whole segment.  The
// B operand of the carry products is built from those registers: the 32x32
// accumulator layout and the B-operand layout of v_mfma_f32_32x32x16_bf16
// both put one column per lane, so only the order of the contraction index
// differs, and the A operand is read from LDS in that same order.
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
constexpr int KTL = 72;    // row length (bf16) of the [channel][token] tiles Kt, Vt
constexpr int KML = 136;   // row length (bf16) of the [token][channel] tiles Km, W0n, Wsn
constexpr int AFL = 68;    // row length (fp32) of A0/T0, A/T
constexpr int TFL = 72;    // row length (bf16) of the scaled T tiles

struct __align__(16) Smem {
    u16 Kt[D * KTL];                                   // keys, [channel][token]
    union {
        u16 Km[CH * KML];                              // keys, [token][channel] (Gram only)
        u16 Vt[D * KTL];                               // values, [channel][token]
    } x;
    union {
        struct { float A0[CH * AFL]; float A1[CH * AFL]; } a;   // A0 -> T0, A -> T (fp32, in place)
        struct { u16 W0n[CH * KML]; u16 Wsn[CH * KML]; } w;     // -W0, -Ws  [token][channel]
    } m;
    struct { u16 T0b[CH * TFL]; u16 Tgb[CH * TFL]; u16 Tb[CH * TFL]; } t;  // T0 diag(b), T diag(b e^g), T diag(b)
    float scratch[2][512];                                                  // 16x16 merge temporaries
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

// 4 + 4 bf16 from two 8-byte aligned LDS addresses
__device__ __forceinline__ bf16x8 lds4x2(const u16 *p0, const u16 *p1) {
    const u32x2 a = *reinterpret_cast<const u32x2 *>(p0);
    const u32x2 b = *reinterpret_cast<const u32x2 *>(p1);
    u32x4 u = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ u16 f2bf(float x) { return __builtin_bit_cast(u16, (__bf16)x); }

__device__ __forceinline__ u16 u4_elem(const uint4 &q, int e) {
    const uint32_t w = e < 2 ? q.x : e < 4 ? q.y : e < 6 ? q.z : q.w;
    return (u16)(w >> (16 * (e & 1)));
}

// Order this wave's LDS writes before its later LDS reads (the lanes of a wave
// run in lockstep, so no workgroup barrier is needed when only this wave reads).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Row of the 32x32 accumulator element held in register r by lane half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// B operand (k-step kb of a 32-row block) from accumulator registers: element e
// of the fragment is accumulator row 8*(2*(kb&1) + e/4) + 4h + (e&3).
__device__ __forceinline__ bf16x8 acc_to_b(const f32x16 &c, int half) {
    const int o = 8 * half;
    return pack8(c[o + 0], c[o + 1], c[o + 2], c[o + 3], c[o + 4], c[o + 5], c[o + 6], c[o + 7]);
}

// Column offset inside a 32-wide block for the A operand that matches acc_to_b:
// elements 0-3 at 16*half + 4h, elements 4-7 at 16*half + 8 + 4h.
__device__ __forceinline__ int perm_col(int half, int h) { return 16 * half + 4 * h; }

__global__ __launch_bounds__(NT, 1) void gdn_build_mfma_kernel(BuildArgs a) {
    __shared__ Smem sm;

    const int th = threadIdx.x;
    const int w = th >> 6, l = th & 63, h = l >> 5, l32 = l & 31;
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
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            st[mb][r] = (!isS && 32 * mb + acc_row(r, h) == col0 + l32) ? 1.0f : 0.0f;
    double ell = 0.0;   // thread 256 (wave 4, lane 0)
    for (int e = th; e < 3 * CH * CH; e += NT) {
        const int t = (e >> 6) & 63, s = e & 63;
        if ((s >> 4) > (t >> 4)) {
            u16 *dst = (e >> 12) == 0 ? sm.t.T0b : (e >> 12) == 1 ? sm.t.Tgb : sm.t.Tb;
            dst[t * TFL + s] = 0;
        }
    }

    const u16 *kp = static_cast<const u16 *>(a.k);
    const u16 *vp = static_cast<const u16 *>(a.v);
    // per thread: token row lt = th / 8, 16 channels from lc = 16 (th % 8) (two 16-byte pieces)
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
        // ---------------- 1. stage keys (Km, Kt) and gates
        *reinterpret_cast<uint4 *>(&sm.x.Km[lt * KML + lc]) = kreg[0];
        *reinterpret_cast<uint4 *>(&sm.x.Km[lt * KML + lc + 8]) = kreg[1];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sm.Kt[(lc + e) * KTL + lt] = u4_elem(kreg[0], e);
            sm.Kt[(lc + 8 + e) * KTL + lt] = u4_elem(kreg[1], e);
        }
        if (th < CH) { sm.la[th] = lareg; sm.beta[th] = breg; }
        const uint4 vkeep0 = vreg[0], vkeep1 = vreg[1];
        if (base + CH < n) fetch(base + CH);     // next chunk's loads fly during this chunk
        __syncthreads();                                                   // B1

        // ---------------- 2. decay prefix (wave 0) | Gram blocks (waves 1-3)
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
            // the segment total of log alpha in fp64 (thread 256 keeps it)
            double gd = (double)sm.la[l];
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) gd += __shfl_xor(gd, o);
            ell += gd;
        } else if (w <= 3) {
#pragma unroll
            for (int r = 0; r < 16; ++r) gacc[r] = 0.f;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const bf16x8 fa = lds8(&sm.x.Km[(32 * gmb + l32) * KML + 16 * kb + 8 * h]);
                const bf16x8 fb = gmb == gnb ? fa : lds8(&sm.x.Km[(32 * gnb + l32) * KML + 16 * kb + 8 * h]);
                gacc = mfma(fa, fb, gacc);
            }
        }
        __syncthreads();                                                   // B2

        // ---------------- 3. A0, A (waves 1-3) ; values to LDS (all)
        if (w >= 1 && w <= 3) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int t = 32 * gmb + acc_row(r, h), s = 32 * gnb + l32;
                float a0 = 0.f, a1 = 0.f;
                if (s < t) {
                    a0 = sm.beta[t] * gacc[r];
                    a1 = a0 * __expf(sm.g[t] - sm.g[s]);
                }
                sm.m.a.A0[t * AFL + s] = a0;
                sm.m.a.A1[t * AFL + s] = a1;
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sm.x.Vt[(lc + e) * KTL + lt] = u4_elem(vkeep0, e);
            sm.x.Vt[(lc + 8 + e) * KTL + lt] = u4_elem(vkeep1, e);
        }
        __syncthreads();                                                   // B3

        // ---------------- 4. UT transform: T0 = (I+A0)^-1, T = (I+A)^-1 in 16x16 blocks,
        //                     writing the bf16 column-scaled forms as blocks become final
        // emit: write the bf16 column-scaled forms of a final T entry (t, s)
        //   matrix 0: T0 diag(beta) -> T0b;  matrix 1: T diag(beta) -> Tb, T diag(beta e^g) -> Tgb
#define HYPIC_EMIT(MAT_, ROW_, COL_, VAL_, SB_, SG_)                          \
    do {                                                                     \
        if ((MAT_) == 0) {                                                   \
            sm.t.T0b[(ROW_) * TFL + (COL_)] = f2bf((VAL_) * (SB_));          \
        } else {                                                             \
            sm.t.Tb[(ROW_) * TFL + (COL_)] = f2bf((VAL_) * (SB_));           \
            sm.t.Tgb[(ROW_) * TFL + (COL_)] = f2bf((VAL_) * (SG_));          \
        }                                                                    \
    } while (0)
        // (a) 16x16 diagonal blocks by forward substitution: wave 0 -> T0, wave 1 -> T
        if (w <= 1) {
            const int mat = w;
            float *M = mat == 0 ? sm.m.a.A0 : sm.m.a.A1;
            const int R = 16 * (l >> 4), j = l & 15;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = 0.f;
#pragma unroll
                for (int s = 0; s < i; ++s) acc += M[(R + i) * AFL + R + s] * x[s];
                x[i] = (i == j) ? 1.0f : (i < j ? 0.0f : -acc);
            }
            const float sb = sm.beta[R + j], sg = sb * sm.eg[R + j];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                M[(R + i) * AFL + R + j] = x[i];
                HYPIC_EMIT(mat, R + i, R + j, x[i], sb, sg);
            }
        }
        __syncthreads();                                                   // B4

        // (b) 16 -> 32: T_10 = -T_11 A_10 T_00, tasks (matrix, half) on waves 0-3
        const int mrow = 4 * (l >> 4), mcol = l & 15;
        if (w < 4) {
            const float *M = (w >> 1) ? sm.m.a.A1 : sm.m.a.A0;
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
            float *M = mat ? sm.m.a.A1 : sm.m.a.A0;
            const int R0 = 32 * (w & 1), R1 = R0 + 16;
            float tc[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) tc[k] = sm.scratch[mat][256 * (w & 1) + k * 16 + mcol];
            const float sb = sm.beta[R0 + mcol], sg = sb * sm.eg[R0 + mcol];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int k = 0; k < 16; ++k) acc += M[(R1 + mrow + r) * AFL + R1 + k] * tc[k];
                M[(R1 + mrow + r) * AFL + R0 + mcol] = -acc;
                HYPIC_EMIT(mat, R1 + mrow + r, R0 + mcol, -acc, sb, sg);
            }
        }
        __syncthreads();                                                   // B6

        // (c) 32 -> 64: T_21 = -T_22 A_21 T_11 on bf16 MFMA, waves 0 and 1
        if (w <= 1) {
            const int mat = w;
            const float *M = mat == 0 ? sm.m.a.A0 : sm.m.a.A1;
            f32x16 tmp;
#pragma unroll
            for (int r = 0; r < 16; ++r) tmp[r] = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const float *ar = &M[(32 + l32) * AFL + 16 * kb + 8 * h];
                const bf16x8 fa = pack8(ar[0], ar[1], ar[2], ar[3], ar[4], ar[5], ar[6], ar[7]);
                const float *bc = &M[(16 * kb + 8 * h) * AFL + l32];
                const bf16x8 fb = pack8(bc[0], bc[AFL], bc[2 * AFL], bc[3 * AFL], bc[4 * AFL], bc[5 * AFL],
                                        bc[6 * AFL], bc[7 * AFL]);
                tmp = mfma(fa, fb, tmp);
            }
            f32x16 o;
#pragma unroll
            for (int r = 0; r < 16; ++r) o[r] = 0.f;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const float *ar = &M[(32 + l32) * AFL + 32 + perm_col(half, h)];
                const bf16x8 fa = pack8(ar[0], ar[1], ar[2], ar[3], ar[8], ar[9], ar[10], ar[11]);
                o = mfma(fa, acc_to_b(tmp, half), o);
            }
            const float sb = sm.beta[l32], sg = sb * sm.eg[l32];
#pragma unroll
            for (int r = 0; r < 16; ++r) HYPIC_EMIT(mat, 32 + acc_row(r, h), l32, -o[r], sb, sg);
        }
#undef HYPIC_EMIT
        __syncthreads();                                                   // B7

        // ---------------- 5. -W0, -Ws (all waves, 2 tiles each) and U (S waves, own columns)
        {
            const u16 *TF = (w >> 2) ? sm.t.Tgb : sm.t.T0b;
            u16 *Wd = (w >> 2) ? sm.m.w.Wsn : sm.m.w.W0n;
            const int mb = (w >> 1) & 1;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int nb = 2 * (w & 1) + q;
                f32x16 c;
#pragma unroll
                for (int r = 0; r < 16; ++r) c[r] = 0.f;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    if (ks >= 2 && mb == 0) break;     // T is lower triangular
                    c = mfma(lds8(&TF[(32 * mb + l32) * TFL + 16 * ks + 8 * h]),
                             lds8(&sm.Kt[(32 * nb + l32) * KTL + 16 * ks + 8 * h]), c);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) Wd[(32 * mb + acc_row(r, h)) * KML + 32 * nb + l32] = f2bf(-c[r]);
            }
        }
        f32x16 acc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
            if (isS) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    if (ks >= 2 && mb == 0) break;
                    acc[mb] = mfma(lds8(&sm.t.Tb[(32 * mb + l32) * TFL + 16 * ks + 8 * h]),
                                   lds8(&sm.x.Vt[(col0 + l32) * KTL + 16 * ks + 8 * h]), acc[mb]);
                }
            }
        }
        __syncthreads();                                                   // B8

        // ---------------- 6. carry: Y = (U) - W . state ; state += K^T diag(.) Y
        {
            const u16 *Wn = isS ? sm.m.w.Wsn : sm.m.w.W0n;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const bf16x8 sb = acc_to_b(st[kb >> 1], kb & 1);
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    const u16 *row = &Wn[(32 * mb + l32) * KML + 32 * (kb >> 1) + perm_col(kb & 1, h)];
                    acc[mb] = mfma(lds4x2(row, row + 8), sb, acc[mb]);
                }
            }
            if (isS) {
                const float eG = sm.eG;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mb][r] *= sm.egr[32 * mb + acc_row(r, h)];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) st[mb][r] *= eG;
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 yb = acc_to_b(acc[s >> 1], s & 1);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    const u16 *row = &sm.Kt[(32 * mb + l32) * KTL + 32 * (s >> 1) + perm_col(s & 1, h)];
                    st[mb] = mfma(lds4x2(row, row + 8), yb, st[mb]);
                }
            }
        }
        __syncthreads();                                                   // B9
    }

    // ---------------- record
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
