// Chunked GDN prefill forward on MFMA with the segment record as a side-output:
// d_k = d_v = 128, bf16 q/k/v, fp32 accumulation, fp64 ell.
//
// What it computes.  Per (segment, head), from a zero state at the segment's
// first token, the recurrence S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} +
// beta_t k_t v_t^T (Gated Delta Networks, podcast companion page, reference 7)
// read out at every token, o_t = S_t^T q_t: the ordinary prefill forward of a
// linear-attention layer.  Beside it, optionally, the segment's record (ell, P, S)
// with T_C = e^ell P (besthub article "Cut First-Token Latency by 3.25x ...",
// paragraph 4: the pair stored at first prefill; paragraph 7: its construction
// costs a small fraction of a forward pass).
//
// Chunk form (64 tokens; g = in-chunk cumulative log decay, G = its total, the
// chunk's start state S_0 = sigma X).  As in the record build (build_mfma.hip):
//   P columns X:  Y = (I + A0)^{-1} (beta . (K X));              X <- X - K^T Y
//   S columns X:  U = (I + A )^{-1} (beta . (V - e^g sigma . (K X)))
//                 X <- e^G X + K^T (e^{G-g} . U)          (sigma bookkeeping as there)
// with A0 = strictlower(beta_t k_t.k_s), A = A0 . e^{g_t - g_s}.  Within the chunk
// S_t = e^{g_t} S_0 + sum_{s<=t} e^{g_t - g_s} k_s u_s^T, so the outputs are
//   O = diag(e^g sigma) (Q X) + Aqk U,   Aqk[t][s] = (q_t.k_s) e^{g_t - g_s} for s <= t
// (the causal mask includes the diagonal: a token's own write is in its output).
//
// Work split: one workgroup per (segment, head), three roles.
//  * S waves 0-3 own 32 state columns each (four fp32 32x32 accumulator tiles,
//    rows swizzled as in the record build).  Per chunk: W = V - e^g sigma (K X) and
//    (Q X)^T in phase b (one pass over X's bf16 operands), the block solve, the
//    update and the chunk's outputs in the next phase a.
//  * P waves 4-7 (records only) own 32 P columns each: W = K X, solve, update.
//  * Four prep waves build the next chunk's factors exactly as the record build's
//    (Gram blocks, blocked inversion, K^T turnaround), plus Aqk.  Without records the
//    queries and Aqk are double-buffered and Aqk's three blocks are computed in phase
//    a on prep waves 1-3 (beside the Gram blocks); with records LDS allows one buffer
//    of each: the queries arrive at the start of the chunk's phase a and Aqk is
//    computed in phase b (block (0,0) on prep wave 0, (1,0) and (1,1) on wave 2).
//    Prep wave 0 also streams k, v (and q) one chunk ahead, double-buffered, spread
//    over both phases: the outputs are stored in phase a, so the values go out in
//    phase a and the keys (and queries) in phase b; with one query buffer the chunk's
//    own queries go out in phase a and the next chunk's keys and values in phase b.
//  * The outputs are formed transposed, (Q X)^T and U^T Aqk^T: the state's bf16
//    operand serves as the A operand of X^T, and a lane then holds one token with
//    four consecutive columns per register group, stored 16 bytes at a time.
// Splitting P and S over separate waves gives every SIMD two independent MFMA
// streams (one S wave, one P wave) beside its prep wave.
// Both barriers of a chunk order LDS only (s_waitcnt lgkmcnt(0); s_barrier): the
// output stores of the S waves are never waited for inside the loop, and prep wave 0
// waits for its own loads (vmcnt) before the barrier that publishes them.
#include "gdn_mfma_common.h"

namespace hypic {
namespace {

enum { SYS_P = 0, SYS_S = 1 };

// 16 bytes per lane from HBM straight into LDS: lane i of the wave lands at dst + 16 i.
// (A non-template helper with the LDS address space explicit: inside the kernel
// template the LDS object's type depends on the template arguments.)
__device__ __forceinline__ void load_lds16(const u16 *src, u16 *dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, kLoadNT);
}

template <bool WITH_P, bool WITH_O>
struct __align__(16) FwdSmem {
    static constexpr bool kWithP = WITH_P;
    static constexpr int NSYS = WITH_P ? 2 : 1;
    static constexpr int kS = NSYS - 1;         // index of the S factors (P at 0 when built)
    // queries: double-buffered like the keys where LDS allows (no P factors), else a
    // single buffer filled at the start of the chunk's phase a
    static constexpr int QBUF = WITH_O ? (WITH_P ? 1 : 2) : 0;
    u16 Km[2][CH * KML];        // keys, token-major, granules swizzled (kmo), double-buffered by parity
    u16 Vm[2][CH * KML];        // values, the same
    u16 Qm[QBUF ? QBUF : 1][QBUF ? CH * KML : 8];   // queries
    u16 Kt[D * KTL];            // keys, channel-major (the update's A operand)
    u16 TB[2][NSYS][2][32 * TBL];  // [parity][system][block]: T_11 diag(beta_1), T_22 diag(beta_2) (P negated)
    u16 H21[2][NSYS][32 * TBL];    // [parity][system]: H_21 (P), -H_21 e^{g_t - g_s} (S)
    // Aqk blocks (0,0), (1,0), (1,1): row t (query), column s (key); by chunk parity
    // when the queries are double-buffered (computed in phase a), else one buffer
    // (computed in phase b)
    static constexpr int ABUF = WITH_O ? (QBUF == 2 ? 2 : 1) : 0;
    u16 Aqk[ABUF ? ABUF : 1][WITH_O ? 3 : 1][32 * TBL];
    float Af[2][32 * AFL];      // diagonal blocks of A0, inverted in place
    float pv[4][2][CH];         // per prep wave: g, beta of the chunk being prepared
    float inv_tmp[4][128];
    float egs[2][CH];           // -e^{g_t} sigma_c
    float egrs[2][CH];          // e^{G - g_t} / sigma_{c+1}
    float rs[2];
    float sig_fin;
    int64_t t0, n;
    int32_t slot, state;
};

// the query buffer of chunk parity b
template <class SM>
__device__ __forceinline__ u16 *qbuf(SM &sm, int b) { return sm.Qm[SM::QBUF == 2 ? b : 0]; }

// the Aqk blocks of chunk parity b (block blk at + 32 TBL blk)
template <class SM>
__device__ __forceinline__ u16 *aqkbuf(SM &sm, int b) { return &sm.Aqk[SM::ABUF == 2 ? b : 0][0][0]; }

// Aqk block blk of the chunk in Km[b] / Qm: A operand = key rows of block am, B operand =
// query rows of block bn, so lane l32 holds query t = 32 bn + l32 and registers hold keys
// s; decayed by e^{g_t - g_s} and masked to s <= t, written row t, column s (bf16).
template <class SM>
__device__ __forceinline__ void prep_aqk(SM &sm, int b, int blk, int pw, int l) {
    const int h = l >> 5, l32 = l & 31;
    const int am = blk == 2 ? 1 : 0, bn = blk == 0 ? 0 : 1;
    const int t = 32 * bn + l32;
    const float gt = sm.pv[pw][0][t];
    bf16x8 fa[8], fb[8];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        fa[kb] = lds8(&sm.Km[b][kmo(32 * am + l32, 2 * kb + h)]);
        fb[kb] = lds8(&qbuf(sm, b)[kmo(32 * bn + l32, 2 * kb + h)]);
    }
    f32x16 g0, g1;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        if (kb & 1) g1 = mfma(fa[kb], fb[kb], kb == 1 ? f32x16{} : g1);
        else g0 = mfma(fa[kb], fb[kb], kb == 0 ? f32x16{} : g0);
    }
    const f32x16 acc = g0 + g1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int s4 = 8 * q + 4 * h;
        const float4 g4 = *reinterpret_cast<const float4 *>(&sm.pv[pw][0][32 * am + s4]);
        const float gs[4] = {g4.x, g4.y, g4.z, g4.w};
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = 32 * am + s4 + e <= t ? acc[4 * q + e] * __expf(gt - gs[e]) : 0.f;
        *reinterpret_cast<u32x2 *>(&aqkbuf(sm, b)[blk * 32 * TBL + l32 * TBL + s4]) =
            u32x2{pack2(x[0], x[1]), pack2(x[2], x[3])};
    }
}

// One state wave: 32 columns (cw) of system SYS for the whole segment.  Outputs (S
// waves with WITH_O) are written for tokens < n; the record columns when `records`.
template <int SYS, bool WITH_O, class SM>
__device__ __forceinline__ void state_wave(SM &sm, const BuildArgs &a, const FwdIO &io, int cw, int64_t t0,
                                           int64_t n, int64_t nc, int head, int64_t rec, bool bad, bool records) {
    constexpr bool OUT = WITH_O && SYS == SYS_S;
    constexpr int SI = SYS == SYS_S ? SM::kS : 0;     // this system's factors in TB, H21
    const int th = threadIdx.x;
    const int col = 32 * cw;
    f32x16 st[4];                    // rows swizzled (physical row p holds channel swz(p))
    bf16x8 wb[2][2];                 // W of the chunk in flight, B operands [token block][half]
    bf16x8 qxb[2][2];                // (OUT) Q X of the chunk in flight, bf16, accumulator order
    {
        const int h = (th & 63) >> 5, l32 = th & 31;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                st[mb][r] = (SYS == SYS_P && swz(32 * mb + acc_row(r, h)) == col + l32) ? 1.0f : 0.0f;
    }
    __syncthreads();                                                // prologue: chunk 0 staged
    for (int64_t i = 0; i <= nc; ++i) {
        int thv = th;
        asm volatile("" : "+v"(thv));
        const int h = (thv & 63) >> 5, l32 = thv & 31;
        // ---- phase a: solve, outputs and update of chunk i - 1
        if (i >= 1) {
            const int b = (int)((i - 1) & 1);
            const int rr = swz(l32) * TBL + 8 * h;
            if (SYS == SYS_S) {
                const float rsc = sm.rs[b];
                if (rsc != 1.0f) {
                    // the pending decay sigma e^G is folded into the state (rare)
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) st[mb][r] *= rsc;
                }
            }
            bf16x8 f0[2], fh[2], f1[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                f0[half] = lds8(&sm.TB[b][SI][0][rr + 16 * half]);
                fh[half] = lds8(&sm.H21[b][SI][rr + 16 * half]);
            }
            f32x16 y1 = mfma(f0[0], wb[0][0], f32x16{});
            y1 = mfma(f0[1], wb[0][1], y1);
            bf16x8 yb[4];
            yb[0] = acc_to_b(y1, 0);
            yb[1] = acc_to_b(y1, 1);
            // W_2 - H_21 Y_1 (H21 carries the sign that makes this a sum), onto W_2 itself
            f32x16 y2;
            {
                const f32x8 w0 = __builtin_convertvector(wb[1][0], f32x8);
                const f32x8 w1 = __builtin_convertvector(wb[1][1], f32x8);
                y2 = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
            }
            y2 = mfma(fh[0], yb[0], y2);
            y2 = mfma(fh[1], yb[1], y2);
#pragma unroll
            for (int half = 0; half < 2; ++half) f1[half] = lds8(&sm.TB[b][SI][1][rr + 16 * half]);
            bf16x8 yu[4];                // (OUT) U as solved, B operands, for the outputs
            if (OUT) { yu[0] = yb[0]; yu[1] = yb[1]; }
            if (SYS == SYS_S) {
                // the update takes e^{G - g} / sigma' . Y
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 e0 = tok4(sm.egrs[b], 0, q, h);
                    y1[4 * q] *= e0.x; y1[4 * q + 1] *= e0.y; y1[4 * q + 2] *= e0.z; y1[4 * q + 3] *= e0.w;
                }
                yb[0] = acc_to_b(y1, 0);
                yb[1] = acc_to_b(y1, 1);
            }
            // X += K^T Y, token steps 0, 1 (they need Y_1 only) beside the Y_2 chain
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                bf16x8 kt[4];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) kt[mb] = lds8(&sm.Kt[swz(32 * mb + l32) * KTL + 16 * s2 + 8 * h]);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) st[mb] = mfma(kt[mb], yb[s2], st[mb]);
            }
            {
                const bf16x8 u0 = acc_to_b(y2, 0), u1 = acc_to_b(y2, 1);
                y2 = mfma(f1[0], u0, f32x16{});
                y2 = mfma(f1[1], u1, y2);
            }
            if (OUT) { yu[2] = acc_to_b(y2, 0); yu[3] = acc_to_b(y2, 1); }
            if (SYS == SYS_S) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 e1 = tok4(sm.egrs[b], 1, q, h);
                    y2[4 * q] *= e1.x; y2[4 * q + 1] *= e1.y; y2[4 * q + 2] *= e1.z; y2[4 * q + 3] *= e1.w;
                }
            }
            yb[2] = acc_to_b(y2, 0);
            yb[3] = acc_to_b(y2, 1);
#pragma unroll
            for (int s2 = 2; s2 < 4; ++s2) {
                bf16x8 kt[4];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) kt[mb] = lds8(&sm.Kt[swz(32 * mb + l32) * KTL + 16 * s2 + 8 * h]);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) st[mb] = mfma(kt[mb], yb[s2], st[mb]);
            }
            if (OUT) {
                // O^T = e^g sigma . (Q X)^T + U^T Aqk^T of chunk i - 1 (after the update, so
                // that only the state, (Q X)^T and U are live beside it): lane = token,
                // registers 4q .. 4q + 3 = columns col + 8q + 4h + 0..3, stored 16 (fp32) or
                // 8 (bf16) contiguous bytes at a time
                const u16 *aq = aqkbuf(sm, b);
                const int ar = l32 * TBL + 8 * h;        // Aqk row t = 32 tb + l32, keys 16 half + 8 h + ..
                const int64_t c0 = (i - 1) * CH;
                const int64_t rem = n - c0;
                const int cl = rem < CH ? (int)rem : CH;
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    const f32x8 q0 = __builtin_convertvector(qxb[tb][0], f32x8);
                    const f32x8 q1 = __builtin_convertvector(qxb[tb][1], f32x8);
                    f32x16 oa = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
                    const float ge = -sm.egs[b][32 * tb + l32];
#pragma unroll
                    for (int r = 0; r < 16; ++r) oa[r] *= ge;
                    if (tb == 0) {
                        oa = mfma(yu[0], lds8(aq + ar), oa);
                        oa = mfma(yu[1], lds8(aq + ar + 16), oa);
                    } else {
                        oa = mfma(yu[0], lds8(aq + 32 * TBL + ar), oa);
                        oa = mfma(yu[1], lds8(aq + 32 * TBL + ar + 16), oa);
                        oa = mfma(yu[2], lds8(aq + 64 * TBL + ar), oa);
                        oa = mfma(yu[3], lds8(aq + 64 * TBL + ar + 16), oa);
                    }
                    const int tok = 32 * tb + l32;
                    if (tok < cl) {
                        const int64_t ob = (t0 + c0 + tok) * io.o_st + (int64_t)head * io.o_sh + col + 4 * h;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            if (io.o_bf16)
                                *reinterpret_cast<u32x2 *>(&static_cast<u16 *>(io.o)[ob + 8 * q]) =
                                    u32x2{pack2(oa[4 * q], oa[4 * q + 1]), pack2(oa[4 * q + 2], oa[4 * q + 3])};
                            else
                                *reinterpret_cast<float4 *>(&static_cast<float *>(io.o)[ob + 8 * q]) =
                                    make_float4(oa[4 * q], oa[4 * q + 1], oa[4 * q + 2], oa[4 * q + 3]);
                        }
                    }
                }
            }
        }
        lds_barrier();                                              // a -> b
        // ---- phase b: W (and Q X) of chunk i from the state before it
        if (i < nc) {
            const int b = (int)(i & 1);
            f32x16 z[2], zq[2];
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const bf16x8 sb = acc_to_b(st[kb >> 1], kb & 1);
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    const int o = kmo(swz(32 * mb + l32), 2 * kb + h);
                    z[mb] = mfma(lds8(&sm.Km[b][o]), sb, kb == 0 ? f32x16{} : z[mb]);
                    // (Q X)^T: the state's operand as A (row = column of X), the query
                    // rows as B (one token per lane, in plain order)
                    if (OUT)
                        zq[mb] = mfma(sb, lds8(&qbuf(sm, b)[kmo(32 * mb + l32, 2 * kb + h)]),
                                      kb == 0 ? f32x16{} : zq[mb]);
                }
            }
            if (SYS == SYS_S) {
                // W = V - e^g sigma . (K X): scale, then add V turned around on the MFMA
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 e4 = tok4(sm.egs[b], mb, q, h);
                        z[mb][4 * q] *= e4.x; z[mb][4 * q + 1] *= e4.y;
                        z[mb][4 * q + 2] *= e4.z; z[mb][4 * q + 3] *= e4.w;
                    }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8 eye = eye_b(ks, h, l32);
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb)
                        z[mb] = mfma(lds8(&sm.Vm[b][kmo(swz(32 * mb + l32), 4 * cw + 2 * ks + h)]), eye, z[mb]);
                }
            }
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    wb[mb][half] = acc_to_b(z[mb], half);
                    if (OUT) qxb[mb][half] = acc_to_b(zq[mb], half);
                }
        }
        lds_barrier();                                              // b -> next a
    }
    if (records) {
        // physical row p of a tile holds channel swz(p); S = sigma X
        const int h = (th & 63) >> 5, l32 = th & 31;
        float *dst = (SYS == SYS_P ? a.pool_P : a.pool_S) + rec * D * D;
        const float sc = SYS == SYS_P ? 1.0f : sm.sig_fin;
        const float nanv = __int_as_float(0x7fc00000);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dst[(int64_t)swz(32 * mb + acc_row(r, h)) * D + col + l32] = bad ? nanv : st[mb][r] * sc;
    }
}

// threads per workgroup: S waves, P waves (records), prep waves
template <bool WITH_P> struct ChunkThreads { static constexpr int value = WITH_P ? 768 : 512; };

template <bool WITH_P, bool WITH_O>
__global__ __launch_bounds__(ChunkThreads<WITH_P>::value, 1) void gdn_chunk_mfma_kernel(BuildArgs a, FwdIO io) {
    using SM = FwdSmem<WITH_P, WITH_O>;
    constexpr int NS = WITH_P ? 8 : 4;           // state waves
    constexpr int NTT = 64 * (NS + 4);
    constexpr bool records = WITH_P;             // a GDN record needs P
    __shared__ SM sm;

    const int th = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(th >> 6);
    const int head = blockIdx.x % a.H;
    const int seg = blockIdx.x / a.H;

    if (th == 0) {
        const int64_t o0 = a.seg_offsets[seg], o1 = a.seg_offsets[seg + 1];
        const int32_t slot = records ? a.dst_slots[seg] : 0;
        int st = 0;
        if (records && (slot < 0 || slot >= a.num_slots)) st = 1;
        else if (o0 < 0 || o1 < o0 || o1 > a.num_tokens) st = 2;
        if (st == 1) raise_flag(a.err_flag, HYPIC_EFLAG_SLOT_OUT_OF_RANGE);
        if (st == 2) raise_flag(a.err_flag, HYPIC_EFLAG_BAD_OFFSETS);
        sm.t0 = o0; sm.n = o1 - o0; sm.slot = slot; sm.state = st;
    }
    // the upper triangles of the T diag(beta) tiles stay zero for the whole segment
    for (int e = th; e < (int)(sizeof(sm.TB) / 16); e += NTT) reinterpret_cast<u32x4 *>(&sm.TB[0][0][0][0])[e] = u32x4{};
    __syncthreads();
    const int state = sm.state;
    if (state == 1) return;
    // bad offsets: no token range to read or write; the record (if any) becomes NaN
    const int64_t t0 = sm.t0;
    const int64_t n = state == 2 ? 0 : sm.n;
    const int64_t nc = (n + CH - 1) / CH;
    const bool bad = state == 2;
    const int64_t rec = (int64_t)sm.slot * a.H + head;

    if (w < 4) {
        state_wave<SYS_S, WITH_O>(sm, a, io, w, t0, n, nc, head, rec, bad, records);
    } else if (WITH_P && w < 8) {
        state_wave<SYS_P, false>(sm, a, io, w - 4, t0, n, nc, head, rec, bad, records);
    } else {
        // =============================== prep waves ===============================
        __builtin_amdgcn_s_setprio(3);
        const int pw = w - NS;
        const int pl = th & 63;
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
            // ---- prep wave 0: streams keys, values (one chunk ahead) and queries (at
            //      the start of the chunk's phase a); decay factors, ell; in phase b K^T
            //      turned around for tokens 0-31 and, with the records, Aqk block (0,0).
            //      Rows past the segment repeat its last row (finite; their beta is zero,
            //      their outputs unused).
            const u16 *kh = static_cast<const u16 *>(a.k) + t0 * a.k_st + head * a.k_sh;
            const u16 *vh = static_cast<const u16 *>(a.v) + t0 * a.v_st + head * a.v_sh;
            const u16 *qh = WITH_O ? static_cast<const u16 *>(io.q) + t0 * io.q_st + head * io.q_sh : nullptr;
            // (the lane index is made opaque at every use, so that the compiler does not
            // hoist 16 row addresses per stream out of the chunk loop into registers)
#define HYPIC_LOAD_ROWS(SRC, ST, BASE, DST)                                                          \
    do {                                                                                             \
        const int64_t base_ = (BASE), rem_ = n - base_;                                              \
        const int cl_ = rem_ < CH ? (int)rem_ : CH;                                                  \
        const u16 *src_ = (SRC) + base_ * (ST);                                                      \
        int lr_ = pl;                                                                                \
        asm volatile("" : "+v"(lr_));                                                                \
        const int r_ = lr_ >> 4, p_ = lr_ & 15;                                                      \
        _Pragma("unroll") for (int u_ = 0; u_ < 16; ++u_) {                                          \
            const int t_ = 4 * u_ + r_, ts_ = t_ < cl_ ? t_ : cl_ - 1;                               \
            load_lds16(src_ + ts_ * (ST) + 8 * (p_ ^ (t_ & 15)), &(DST)[4 * u_ * KML]);              \
        }                                                                                            \
    } while (0)
            double ell = 0.0;
            float sig = 1.0f;
            if (pl == 0) sm.sig_fin = 1.0f;
            if (nc > 0) {
                HYPIC_LOAD_ROWS(kh, a.k_st, 0, sm.Km[0]);
                HYPIC_LOAD_ROWS(vh, a.v_st, 0, sm.Vm[0]);
                if (SM::QBUF == 2) HYPIC_LOAD_ROWS(qh, io.q_st, 0, qbuf(sm, 0));
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            __syncthreads();                                        // prologue: chunk 0 staged
            for (int64_t i = 0; i <= nc; ++i) {
                int thv = th;
                asm volatile("" : "+v"(thv));
                const int l = thv & 63;
                if (i < nc) {
                    const int b = (int)(i & 1);
                    const float la_i = lar, b_i = br;
                    // Loads are spread over both phases (the outputs are stored in phase a):
                    // one query buffer: this chunk's queries now (read in phase b), the next
                    // chunk's keys and values in phase b; otherwise the next chunk's values
                    // now, its keys (and queries) in phase b.
                    if (SM::QBUF == 1) HYPIC_LOAD_ROWS(qh, io.q_st, i * CH, qbuf(sm, 0));
                    else if (i + 1 < nc) HYPIC_LOAD_ROWS(vh, a.v_st, (i + 1) * CH, sm.Vm[b ^ 1]);
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
                    if (SM::QBUF == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // queries landed
                }
                lds_barrier();                                      // a -> b
                if (i + 1 < nc) {
                    const int nb = (int)(i & 1) ^ 1;
                    HYPIC_LOAD_ROWS(kh, a.k_st, (i + 1) * CH, sm.Km[nb]);
                    if (SM::QBUF == 1) HYPIC_LOAD_ROWS(vh, a.v_st, (i + 1) * CH, sm.Vm[nb]);
                    if (SM::QBUF == 2) HYPIC_LOAD_ROWS(qh, io.q_st, (i + 1) * CH, qbuf(sm, nb));
                    HYPIC_FETCH_G((i + 1) * CH);
                }
                if (i < nc) {
                    prep_kt(sm, (int)(i & 1), 0, l);
                    if (SM::ABUF == 1) prep_aqk(sm, (int)(i & 1), 0, 0, l);
                }
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // chunk i + 1 has landed
                lds_barrier();                                      // b -> next a
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) ell += __shfl_xor(ell, o);
            if (records && pl == 0) a.pool_ell[rec] = bad ? __int_as_float(0x7fc00000) : (float)ell;
#undef HYPIC_LOAD_ROWS
        } else {
            // ---- prep waves 1-3: a Gram block in phase a (waves 1 and 3 the diagonal blocks,
            //      which they also start inverting, wave 2 H_21; without the records also
            //      Aqk blocks (0,0), (1,0), (1,1)); in phase b waves 1 and 3 finish their
            //      block's inverse, and wave 2 turns K^T around for tokens 32-63 and, with
            //      the records, computes Aqk blocks (1,0) and (1,1)
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
                        prep_invert1<WITH_P>(inv_ctx(sm, b, pw >> 1, pw), l);
                    }
                    // double-buffered Aqk: this chunk's blocks (0,0), (1,0), (1,1) on waves 1, 2, 3
                    if (SM::ABUF == 2) prep_aqk(sm, b, pw - 1, pw, l);
                }
                lds_barrier();                                      // a -> b
                if (i + 1 < nc) HYPIC_FETCH_G((i + 1) * CH);
                if (i < nc && pw != 2) prep_invert2<WITH_P>(inv_ctx(sm, (int)(i & 1), pw >> 1, pw), l);
                if (i < nc && pw == 2) {
                    prep_kt(sm, (int)(i & 1), 1, l);
                    if (SM::ABUF == 1) {
                        prep_aqk(sm, (int)(i & 1), 1, 2, l);
                        prep_aqk(sm, (int)(i & 1), 2, 2, l);
                    }
                }
                lds_barrier();                                      // b -> next a
            }
        }
#undef HYPIC_FETCH_G
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_build_mfma(const BuildArgs &a, hipStream_t stream, bool *taken);

// The chunked forward (outputs) with or without the records, for GDN with bf16 k/v
// and q at d_k = d_v = 128 with 16-byte aligned rows; the records alone go to the
// record build (build_mfma.hip), whose single-role state waves keep more of the
// matrix pipe busy than separate P and S waves do.
// *taken = false: the shapes are not the kernels' (nothing launched).
hipError_t launch_chunk_mfma(const BuildArgs &a, const FwdIO &io, bool records, bool outputs, hipStream_t stream,
                             bool *taken) {
    *taken = false;
    if (!outputs) return records ? launch_build_mfma(a, stream, taken) : hipSuccess;
    if (a.family != HYPIC_GDN || a.kv_dtype != HYPIC_BF16 || a.dk != 128 || a.dv != 128) return hipSuccess;
    if (!aligned16(a.k) || !aligned16(a.v) || (a.k_st % 8) || (a.k_sh % 8) || (a.v_st % 8) || (a.v_sh % 8))
        return hipSuccess;
    if (outputs && (!aligned16(io.q) || (io.q_st % 8) || (io.q_sh % 8) || !aligned16(io.o) || (io.o_st % 8) ||
                    (io.o_sh % 8)))
        return hipSuccess;
    *taken = true;
    const dim3 grid((unsigned)((int64_t)a.num_segments * a.H));
    if (records) hipLaunchKernelGGL((gdn_chunk_mfma_kernel<true, true>), grid, dim3(768), 0, stream, a, io);
    else hipLaunchKernelGGL((gdn_chunk_mfma_kernel<false, true>), grid, dim3(512), 0, stream, a, io);
    return hipGetLastError();
}

}  // namespace hypic
